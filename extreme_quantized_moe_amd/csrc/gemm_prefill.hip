// Matrix-core (prefill) path of the routed W3A16 + low-rank grouped GEMM.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up).  MiLo Kernel: int3 x fp16 GEMM
// with fused dequantization; asynchronous global loads overlap memory with
// compute.  MiLo Algorithm: W_out = W_quant + U V.
//
// Grid: x = n-tile groups (fastest), y = row tiles of BM rows (128 where
// experts average 256 rows or more, else 64), so the blocks that run together
// share activation rows (L2 hits) while the weights stream.
// Block = BM rows of one expert (pairs in sorted order) x 4 waves.  Each wave
// owns one 64-wide output tile of one weight family (SWIGLU: waves (W1, W3) x
// two n-tiles; otherwise four n-tiles of the one family), so every packed
// weight tile is read and dequantized by exactly one wave.  Activation rows
// go straight from global memory into LDS (global_load_lds_dwordx4: BM rows
// x 128 K, double buffered, 16-byte chunks XOR-swizzled per row against bank
// conflicts) and are shared by the four waves; the next K block's
// activations (into LDS) and weights (into registers) load while the current
// one is computed.  Weights are dequantized in registers (int3 pair
// extraction, then packed fp16: subtract the offset, one fused multiply-add
// by the scale with -z s) and multiplied on v_mfma_f32_16x16x32_f16 with fp32
// accumulation; each K block is one branch-free region the scheduler
// interleaves, issued at raised wave priority.
// Epilogue: low-rank term as two more matrix-core K-steps per 32 ranks, then
// SWIGLU through LDS, or fp16 store, or route-weighted fp32 scatter.
#include "gemm_common.hpp"

namespace milo {

constexpr int kXStride = kTileK;         // LDS row stride in halves (256 B; chunks swizzled)
constexpr int kExStride = 68;            // floats per row of the SwiGLU exchange
// LDS of a BM-row block: two staging buffers, or the SwiGLU exchange
constexpr size_t prefill_lds(int bm) {
  return 2 * bm * kExStride * 4 > 2 * bm * kXStride * 2 ? (size_t)2 * bm * kExStride * 4 : (size_t)2 * bm * kXStride * 2;
}

// Weight dequantization in packed fp16: from the extracted pair h = (off + q)
// (exact), q = h - off is exact, and (q - z) s = fma(q, s, -z s) with -z s
// rounded to fp16 once per group: two packed instructions per pair.  Error
// per weight at most half an fp16 ulp of z s plus half an ulp of the result.
struct GroupConstPk {
  f16x2 s, nzs;
};

// -z s as one fp16 multiply: the product of two fp16 values is exact in fp32,
// so this is the same correctly rounded value as rounding the fp32 product.
__device__ __forceinline__ GroupConstPk group_const_pk(uint32_t szword) {
  const f16x2 sz = __builtin_bit_cast(f16x2, szword);   // (s, z)
  const _Float16 nz = -(sz[1] * sz[0]);
  GroupConstPk g;
  g.s = f16x2{sz[0], sz[0]};
  g.nzs = f16x2{nz, nz};
  return g;
}

__device__ __forceinline__ f16x8 dequant_step_pk(const uint32_t h[16], int step, const GroupConstPk& g) {
  const f16x2 off64 = {(_Float16)64.f, (_Float16)64.f}, off8 = {(_Float16)8.f, (_Float16)8.f};
  u32x4 u;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int pi = 4 * step + v;
    const f16x2 q = __builtin_bit_cast(f16x2, h[pi]) - (pair_offset(pi) == 64 ? off64 : off8);
    u[v] = __builtin_bit_cast(uint32_t, q * g.s + g.nzs);
  }
  return __builtin_bit_cast(f16x8, u);
}

template <int NW, bool LRQ, int BM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_prefill_kernel(GemmArgs a) {
  constexpr int kMT = BM / 16;            // m-tiles per wave
  constexpr int kXBuf = BM * kXStride;     // halves per staging buffer
  extern __shared__ __align__(16) uint16_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const CodeConsts kc = make_code_consts();
  RowTile rt;
  if (!find_row_tile(a.offsets, a.num_experts, a.pre_min_rows, BM, blockIdx.y, a.rp ? a.rank[0] : nullptr,
                     a.rp ? a.rank[1] : nullptr, &rt))
    return;
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  const int f = (NW == 2) ? (wave & 1) : 0;
  const int nt = (NW == 2) ? (2 * blockIdx.x + (wave >> 1)) : (4 * blockIdx.x + wave);
  const bool wave_on = nt < a.n_tiles;

  // ---- activation staging, global memory -> LDS without registers: per K
  // block a wave issues BM / 16 loads of 1 KB, load j filling rows 16 j + 4 wave ..
  // + 3 (lane l: row + l / 16, 16-byte slot l % 16).  Slot p of row r holds
  // column chunk p ^ (r % 16), so a fragment read (16 rows, one chunk) hits
  // 16 different slots.  Rows past the expert's count read its first row
  // instead: they only feed output rows that are not stored.
  const int srow = 4 * wave + (lane >> 4);
  int xrow[BM / 16];
#pragma unroll
  for (int j = 0; j < BM / 16; ++j) {
    const int m = m0 + srow + 16 * j;
    const int i = base + (m < M ? m : m0);
    xrow[j] = a.gather_div > 0 ? a.sorted_pairs[i] / a.gather_div : i;
  }
  const uint16_t* xcol = a.x + 8 * ((lane & 15) ^ (srow & 15));
  auto stage_x = [&](int kb, int buf) {
#pragma unroll
    for (int j = 0; j < BM / 16; ++j)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(xcol + (size_t)xrow[j] * a.K + (size_t)kb * kTileK),
          (__attribute__((address_space(3))) void*)(lds + buf * kXBuf + (16 * j + 4 * wave) * kXStride), 16, 0, 0);
  };
  // fragment of K step s: row lane % 16 of each m-tile, chunk 4 s + lane / 16
  int xoff[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) xoff[s4] = (lane & 15) * kXStride + 8 * ((4 * s4 + (lane >> 4)) ^ (lane & 15));

  // ---- weights of this wave
  const uint32_t* tbase = a.packed[f] + e * a.words_per_expert + (size_t)(wave_on ? nt : 0) * a.kblocks * kTileWords;
  const uint32_t* sbase = a.sz[f] + e * a.sz_per_expert + (size_t)(wave_on ? nt : 0) * a.kblocks * kTileSzWords;
  u32x4 wq[3], wz[2], nq[3], nz[2];
  auto load_w = [&](int kb, u32x4 (&q)[3], u32x4 (&z)[2]) {
    const uint32_t* tp = tbase + (size_t)kb * kTileWords;
    const uint32_t* sp = sbase + (size_t)kb * kTileSzWords + 8 * (lane & 15);
    q[0] = *(const u32x4*)(tp + 4 * lane);
    q[1] = *(const u32x4*)(tp + 256 + 4 * lane);
    q[2] = *(const u32x4*)(tp + 512 + 4 * lane);
    z[0] = *(const u32x4*)(sp);
    z[1] = *(const u32x4*)(sp + 4);
  };

  f32x4 acc[kMT][4];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  stage_x(0, 0);
  if (wave_on) load_w(0, wq, wz);
  __syncthreads();   // waits for the staging loads (vmcnt) first

  // B operands of K step s of the current block, from the lane's triplets
  auto dequant = [&](f16x8 (&wf)[4], int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h[16];
      extract_triplet(wq[0][i], wq[1][i], wq[2][i], h, kc);
      const int idx = 2 * i + (s >> 1);
      const GroupConstPk gc = group_const_pk(idx < 4 ? wz[0][idx] : wz[1][idx - 4]);
      wf[i] = dequant_step_pk(h, s, gc);
    }
  };

  // Each K block is one straight-line region (the prefetch indices are
  // clamped instead of branched on; the last block re-loads its own data),
  // so the scheduler can overlap a step's dequantization with the previous
  // step's products.
  const int KB = a.kblocks;
  if (wave_on) {
    for (int kb = 0; kb < KB; ++kb) {
      const int buf = kb & 1;
      const int kn = kb + 1 < KB ? kb + 1 : kb;
      stage_x(kn, buf ^ 1);
      // one weight family: the next block's weights load ahead of this
      // block's work (a second register set); two families keep one set
      // (no registers to spare) and load after the last step's dequantization
      if constexpr (NW == 1) {
        load_w(kn, nq, nz);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint16_t* xb = lds + buf * kXBuf;
      // raised wave priority while a block's products issue, back to normal
      // at the barrier: the two waves sharing a SIMD drift out of phase, one
      // issuing products while the other waits at its barrier or on loads
      // (measured: gate/up 93.5 -> 84.6 us on 64-row tiles, -1.6 % on 128)
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 wf[4];
        dequant(wf, s);
        if (NW == 2 && s == 3) load_w(kn, wq, wz);   // the codes of this block are consumed
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const f16x8 xa = *(const f16x8*)(xb + xoff[s] + mt * 16 * kXStride);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][i] = mfma16x16x32(xa, wf[i], acc[mt][i]);
        }
      }
      if constexpr (NW == 1) {
#pragma unroll
        for (int j = 0; j < 3; ++j) wq[j] = nq[j];
        wz[0] = nz[0];
        wz[1] = nz[1];
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();   // waits for the staging loads (vmcnt) first
    }
  } else {
    // no output tile: only the share of the activation staging
    for (int kb = 0; kb < KB; ++kb) {
      stage_x(kb + 1 < KB ? kb + 1 : kb, (kb & 1) ^ 1);
      __syncthreads();
    }
  }

  // ---- low-rank term: (x V^T) U^T as extra K steps (int3 U: the lane's
  // triplet of each 32-rank U tile is its B operand for the four row groups)
  if (wave_on && a.rp > 0) {
    const int RW = a.n_w * a.rp;
    const int rk = rt.rank(f);
    u32x4 usz = {0u, 0u, 0u, 0u};
    if constexpr (LRQ) usz = *(const u32x4*)(a.Usz[f] + (size_t)e * a.N + nt * kTileRows + 4 * (lane & 15));
    for (int s2 = 0; s2 < a.rp / 32; ++s2) {
      const int j0 = 32 * s2 + 8 * (lane >> 4);
      f16x8 ub[4];
      if constexpr (LRQ) {
        const uint32_t* up = a.Uq[f] + e * a.uq_per_expert + ((size_t)nt * (a.rp / 32) + s2) * 192 + lane;
        uint32_t h[16];
        extract_triplet(up[0], up[64], up[128], h, kc);
#pragma unroll
        for (int i = 0; i < 4; ++i) ub[i] = j0 < rk ? dequant_step(h, i, group_const(usz[i])) : f16x8{};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nt * kTileRows + 16 * i + (lane & 15);
          ub[i] = j0 < rk ? *(const f16x8*)(a.U[f] + ((size_t)e * a.N + n) * a.max_rank + j0) : f16x8{};
        }
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int m = m0 + mt * 16 + (lane & 15);
        const f16x8 ta = m < M ? *(const f16x8*)(a.T + (size_t)(base + m) * RW + f * a.rp + j0) : f16x8{};
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = mfma16x16x32(ta, ub[i], acc[mt][i]);
      }
    }
  }

  // ---- epilogue
  if (NW == 2) {
    // waves with f == 1 (W3) hand their tile to the partner wave (wave - 1)
    // rows padded to kExStride floats: the four row groups of a wave's
    // accumulators then fall on different LDS banks
    float* ex = (float*)lds + (wave >> 1) * (BM * kExStride);
    if (wave_on && f == 1) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ex[(mt * 16 + 4 * (lane >> 4) + r) * kExStride + 16 * i + (lane & 15)] = acc[mt][i][r];
    }
    __syncthreads();
    if (!wave_on || f == 1) return;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = mt * 16 + 4 * (lane >> 4) + r;
        if (m0 + mm >= M) continue;
        uint16_t* yrow = (uint16_t*)a.y + (size_t)(base + m0 + mm) * a.N + nt * kTileRows;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = 16 * i + (lane & 15);
          const float h3 = ex[mm * kExStride + n];
          yrow[n] = float_to_half_bits(silu(acc[mt][i][r]) * h3);
        }
      }
    return;
  }
  if (!wave_on) return;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = mt * 16 + 4 * (lane >> 4) + r;
      if (m0 + mm >= M) continue;
      const int i_pair = base + m0 + mm;
      if (a.epilogue == MILO_EPI_ROUTE_SCALE) {
        const int s = a.sorted_pairs[i_pair];
        const float w = a.slot_w[s];
        float* yrow = (float*)a.y + (size_t)s * a.N + nt * kTileRows;
#pragma unroll
        for (int i = 0; i < 4; ++i) yrow[16 * i + (lane & 15)] = acc[mt][i][r] * w;
      } else {
        uint16_t* yrow = (uint16_t*)a.y + (size_t)i_pair * a.N + nt * kTileRows;
#pragma unroll
        for (int i = 0; i < 4; ++i) yrow[16 * i + (lane & 15)] = float_to_half_bits(acc[mt][i][r]);
      }
    }
}


int32_t launch_gemm_prefill(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  if (!p.pre_launch) return MILO_OK;
  GemmArgs a = make_gemm_args(d, p, ws);
  // 128-row tiles where experts average 256 rows or more, else 64-row tiles
  // (less padding and twice the blocks for mid-sized experts)
  const dim3 grid(d->n_w == 2 ? (p.n_tiles + 1) / 2 : (p.n_tiles + 3) / 4, p.pre_tiles);
  if (p.pre_bm == 128) {
    const size_t lds = prefill_lds(128);
    if (d->n_w == 2) {
      if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<2, true, 128>), grid, dim3(256), lds, st, a);
      else hipLaunchKernelGGL((gemm_prefill_kernel<2, false, 128>), grid, dim3(256), lds, st, a);
    } else {
      if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<1, true, 128>), grid, dim3(256), lds, st, a);
      else hipLaunchKernelGGL((gemm_prefill_kernel<1, false, 128>), grid, dim3(256), lds, st, a);
    }
  } else {
    const size_t lds = prefill_lds(64);
    if (d->n_w == 2) {
      if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<2, true, 64>), grid, dim3(256), lds, st, a);
      else hipLaunchKernelGGL((gemm_prefill_kernel<2, false, 64>), grid, dim3(256), lds, st, a);
    } else {
      if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<1, true, 64>), grid, dim3(256), lds, st, a);
      else hipLaunchKernelGGL((gemm_prefill_kernel<1, false, 64>), grid, dim3(256), lds, st, a);
    }
  }
  return hip_status(hipGetLastError(), "gemm_prefill_kernel launch");
}

}  // namespace milo
