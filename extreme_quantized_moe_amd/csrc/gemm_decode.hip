// Small-M (decode) path of the routed W3A16 + low-rank grouped GEMM.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up).  MiLo Kernel: an int3 x fp16
// GEMM with the dequantization fused into the kernel (no separate dequantized
// copy of the weights in memory), and asynchronous global loads to hide
// memory latency.  MiLo Algorithm: W_out = W_quant + U V.
//
// At decode an expert sees a handful of rows, so the kernel streams the
// packed weights once from HBM: block (n-tile of 64 output features, expert,
// K split) = 4 waves, wave w takes the 128-wide K blocks w, w+4, ... of the
// block's range.  Per K block a wave issues three 16-byte loads per lane for
// the 64 x 128 codes (one per plane of layout v1) and two for the scale/zero
// words, extracts the int3 pairs in registers, dequantizes them to float16
// and feeds 16x16x32 f16 matrix-core ops with the rows of the expert as the A
// operand (16 rows per m-tile, rows beyond the expert's count are zero).
// Loads of the next K block are issued before the current one is consumed.
// Waves are summed in LDS in wave order, K splits by the last block to finish
// in split order, then the epilogue (low-rank term already added by wave 0 of
// split 0) stores fp16 (NONE / SWIGLU) or scales and scatters fp32
// (ROUTE_SCALE).
#include "gemm_common.hpp"

namespace milo {

struct WTile {
  u32x4 q[3];
  u32x4 z[2];
};

__device__ __forceinline__ void load_wtile(WTile& t, const uint32_t* tp, const uint32_t* sp, int lane) {
  t.q[0] = *(const u32x4*)(tp + 4 * lane);
  t.q[1] = *(const u32x4*)(tp + 256 + 4 * lane);
  t.q[2] = *(const u32x4*)(tp + 512 + 4 * lane);
  const uint32_t* s = sp + 8 * (lane & 15);
  t.z[0] = *(const u32x4*)(s);
  t.z[1] = *(const u32x4*)(s + 4);
}

// sz word for row group i and group g of the tile: index 2 i + g of the lane's 8
__device__ __forceinline__ uint32_t sz_word(const WTile& t, int i, int g) {
  const int idx = 2 * i + g;
  return idx < 4 ? t.z[0][idx] : t.z[1][idx - 4];
}

template <int MT, int NW>
__device__ __forceinline__ void consume_tile(const WTile& t, const f16x8 (&xa)[MT][4],
                                             f32x4 (&acc)[MT][4], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h[16];
    extract_triplet(t.q[0][i], t.q[1][i], t.q[2][i], h);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const GroupConst gc = group_const(sz_word(t, i, g));
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const int step = 2 * g + ss;
        const f16x8 wb = dequant_step(h, step, gc);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][i] = mfma16x16x32(xa[mt][step], wb, acc[mt][i]);
      }
    }
  }
}

template <int MT, int NW>
__global__ void __launch_bounds__(256) gemm_decode_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = blockIdx.x, e = blockIdx.y, ks = blockIdx.z;
  const int base = a.offsets[e];
  const int M = a.offsets[e + 1] - base;
  if (M == 0 || M > a.dec_max_rows) return;

  // A operand (rows of the expert) pointers
  const uint16_t* xp[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    xok[mt] = m < M;
    int xr = 0;
    if (xok[mt]) xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
    xp[mt] = a.x + (size_t)xr * a.K + 8 * (lane >> 4);
  }

  f32x4 acc[NW][MT][4];
#pragma unroll
  for (int f = 0; f < NW; ++f)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kb0 = (int)((int64_t)a.kblocks * ks / a.ksplit);
  const int kb1 = (int)((int64_t)a.kblocks * (ks + 1) / a.ksplit);
  const uint32_t* tbase[NW];
  const uint32_t* sbase[NW];
#pragma unroll
  for (int f = 0; f < NW; ++f) {
    tbase[f] = a.packed[f] + e * a.words_per_expert + (size_t)nt * a.kblocks * kTileWords;
    sbase[f] = a.sz[f] + e * a.sz_per_expert + (size_t)nt * a.kblocks * kTileSzWords;
  }

  int kb = kb0 + wave;
  WTile cur[NW], nxt[NW];
  if (kb < kb1) {
#pragma unroll
    for (int f = 0; f < NW; ++f)
      load_wtile(cur[f], tbase[f] + (size_t)kb * kTileWords, sbase[f] + (size_t)kb * kTileSzWords, lane);
  }
  for (; kb < kb1; kb += 4) {
    const int kn = kb + 4;
    if (kn < kb1) {
#pragma unroll
      for (int f = 0; f < NW; ++f)
        load_wtile(nxt[f], tbase[f] + (size_t)kn * kTileWords, sbase[f] + (size_t)kn * kTileSzWords, lane);
    }
    f16x8 xa[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xa[mt][s] = xok[mt] ? *(const f16x8*)(xp[mt] + (size_t)kb * kTileK + 32 * s) : f16x8{};
#pragma unroll
    for (int f = 0; f < NW; ++f) consume_tile<MT, NW>(cur[f], xa, acc[f], lane);
#pragma unroll
    for (int f = 0; f < NW; ++f) cur[f] = nxt[f];
  }

  // low-rank term (x V^T) U^T: two more K steps per 32 ranks, added once
  if (wave == 0 && ks == 0 && a.rp > 0) {
    const int RW = a.n_w * a.rp;
#pragma unroll
    for (int f = 0; f < NW; ++f) {
      const int rk = a.rank[f][e];
      for (int s2 = 0; s2 < a.rp / 32; ++s2) {
        const int j0 = 32 * s2 + 8 * (lane >> 4);
        f16x8 ta[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + (lane & 15);
          ta[mt] = m < M ? *(const f16x8*)(a.T + (size_t)(base + m) * RW + f * a.rp + j0) : f16x8{};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nt * kTileRows + 16 * i + (lane & 15);
          f16x8 ub = f16x8{};
          if (j0 < rk) ub = *(const f16x8*)(a.U[f] + ((size_t)e * a.N + n) * a.max_rank + j0);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[f][mt][i] = mfma16x16x32(ta[mt], ub, acc[f][mt][i]);
        }
      }
    }
  }

  // ---- cross-wave reduction (wave order), one weight family at a time
  constexpr int kOut = MT * 16 * 64;       // outputs per family per block
  constexpr int kPer = kOut / 256;         // per thread
  __shared__ float red[4][kOut];
  __shared__ int is_last;
  float res[NW][kPer];
#pragma unroll
  for (int f = 0; f < NW; ++f) {
    if (f) __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mt * 16 + 4 * (lane >> 4) + r, n = 16 * i + (lane & 15);
          red[wave][m * 64 + n] = acc[f][mt][i][r];
        }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int o = threadIdx.x + 256 * c;
      res[f][c] = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
    }
  }

  // ---- split-K: last block to finish sums the splits in split order
  if (a.ksplit > 1) {
    const size_t slot = ((size_t)e * a.n_tiles + nt);
    float* mine = a.part + ((size_t)ks * a.num_experts * a.n_tiles + slot) * (NW * kOut);
#pragma unroll
    for (int f = 0; f < NW; ++f)
#pragma unroll
      for (int c = 0; c < kPer; ++c) mine[f * kOut + threadIdx.x + 256 * c] = res[f][c];
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(&a.cnt[slot], 1);
      is_last = (prev == a.ksplit - 1);
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
#pragma unroll
    for (int f = 0; f < NW; ++f)
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        float v = 0.f;
        for (int s = 0; s < a.ksplit; ++s)
          v += __builtin_nontemporal_load(
              a.part + ((size_t)s * a.num_experts * a.n_tiles + slot) * (NW * kOut) + f * kOut +
              threadIdx.x + 256 * c);
        res[f][c] = v;
      }
    if (threadIdx.x == 0) a.cnt[slot] = 0;
  }

  // ---- epilogue
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const int o = threadIdx.x + 256 * c;
    const int m = o >> 6, n = o & 63;
    if (m >= M) continue;
    const int i = base + m;
    const int col = nt * kTileRows + n;
    if (a.epilogue == MILO_EPI_ROUTE_SCALE) {
      const int s = a.sorted_pairs[i];
      ((float*)a.y)[(size_t)s * a.N + col] = res[0][c] * a.slot_w[s];
    } else {
      float v = res[0][c];
      if (NW == 2) v = silu(v) * res[NW - 1][c];
      ((uint16_t*)a.y)[(size_t)i * a.N + col] = float_to_half_bits(v);
    }
  }
}

template <int MT>
static void launch_mt(const GemmArgs& a, dim3 grid, hipStream_t st) {
  if (a.n_w == 2)
    hipLaunchKernelGGL((gemm_decode_kernel<MT, 2>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<MT, 1>), grid, dim3(256), 0, st, a);
}

GemmArgs make_gemm_args(const milo_gemm_desc* d, const GemmPlan& p, char* ws);

int32_t launch_gemm_decode(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  if (p.dec_mt == 0) return MILO_OK;
  GemmArgs a = make_gemm_args(d, p, ws);
  a.part = (float*)(ws + p.off_dec_part);
  a.cnt = (int32_t*)(ws + p.off_dec_cnt);
  dim3 grid(p.n_tiles, d->num_experts, p.dec_ksplit);
  switch (p.dec_mt) {
    case 1: launch_mt<1>(a, grid, st); break;
    case 2: launch_mt<2>(a, grid, st); break;
    case 4: launch_mt<4>(a, grid, st); break;
    default: set_error("internal: bad m-tile count %d", p.dec_mt); return MILO_ERR_ARG;
  }
  return hip_status(hipGetLastError(), "gemm_decode_kernel launch");
}

}  // namespace milo
