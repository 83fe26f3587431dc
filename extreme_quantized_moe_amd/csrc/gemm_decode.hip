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
// the 64 x 128 codes (one per plane of layout v1), two for the scale/zero
// words, four per 16-row m-tile for the activation fragments and four per
// m-tile for the per-group activation sums; these loads run DEPTH-1 K blocks
// ahead of the block being consumed (a register ring).
//
// Dequantization is folded out of the inner product.  The extraction turns a
// pair of int3 codes into two exact float16 values off + q (off = 64 or 8,
// one v_and_or_b32 per pair), and the matrix cores compute, per 64-wide group
// g, P = sum_k x_k (off_k + q_k) starting from the accumulator value
// -(sum_k x_k off_k) - z sum_k x_k (both sums precomputed per row and group by
// the pre-pass), so that P = sum_k x_k (q_k - z) up to fp32 rounding; then
// y += s P in fp32.  No weight is rounded to float16.  The expert's rows are
// the A operand (16 per m-tile, rows beyond the expert's count are zero) and
// the codes the B operand.  Waves are summed in LDS in wave order.  With one
// K split the block applies the epilogue itself; with several, each split
// stores its sum and gemm_decode_reduce adds the splits in split order and
// applies the epilogue (no cross-block synchronisation inside a kernel).  The
// low-rank term is added by wave 0 of split 0.
#include "gemm_common.hpp"

namespace milo {

struct WTile {
  u32x4 q[3];
  u32x4 z[2];
};

template <int MT, int NW>
struct Stage {
  WTile w[NW];
  f16x8 x[MT][4];
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

template <int MT>
__device__ __forceinline__ void consume_tile(const WTile& t, const f16x8 (&xa)[MT][4],
                                             const f32x4 (&xs)[2][MT], const f32x4 (&xo)[2][MT],
                                             f32x4 (&acc)[MT][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h[16];
    extract_triplet(t.q[0][i], t.q[1][i], t.q[2][i], h);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t w = sz_word(t, i, g);
      const float s = half_bits_to_float(w & 0xFFFFu);
      const float z = half_bits_to_float(w >> 16);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_fmaf(-z, xs[g][mt][r], -xo[g][mt][r]);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const int step = 2 * g + ss;
          const u32x4 u = {h[4 * step], h[4 * step + 1], h[4 * step + 2], h[4 * step + 3]};
          p = mfma16x16x32(xa[mt][step], __builtin_bit_cast(f16x8, u), p);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][i][r] = __builtin_fmaf(s, p[r], acc[mt][i][r]);
      }
    }
  }
}

template <int MT, int NW>
struct DecodeCtx {
  const uint32_t* tbase[NW];
  const uint32_t* sbase[NW];
  const uint16_t* xp[MT];
  const float* lds_xs;    // [local group][16 MT rows], then xo at + lds_half
  int lds_half;
  int g0;                 // first group of the block's K range
  bool xok[MT];
  int lane;

  __device__ __forceinline__ void load(Stage<MT, NW>& S, int kb) const {
#pragma unroll
    for (int f = 0; f < NW; ++f)
      load_wtile(S.w[f], tbase[f] + (size_t)kb * kTileWords, sbase[f] + (size_t)kb * kTileSzWords, lane);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        S.x[mt][s] = xok[mt] ? *(const f16x8*)(xp[mt] + (size_t)kb * kTileK + 32 * s) : f16x8{};
  }
  __device__ __forceinline__ void consume(const Stage<MT, NW>& S, int kb, f32x4 (&acc)[NW][MT][4]) const {
    f32x4 xs[2][MT], xo[2][MT];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float* q = lds_xs + (2 * kb + g - g0) * (16 * MT) + mt * 16 + 4 * (lane >> 4);
        xs[g][mt] = *(const f32x4*)q;
        xo[g][mt] = *(const f32x4*)(q + lds_half);
      }
#pragma unroll
    for (int f = 0; f < NW; ++f) consume_tile<MT>(S.w[f], S.x, xs, xo, acc[f]);
  }
};

// Final values -> outputs.  res[f][c] holds output (m, n) = (o >> 6, o & 63)
// with o = threadIdx.x + 256 c of the 64-wide n-tile nt of expert e.
template <int NW, int KPER>
__device__ __forceinline__ void decode_epilogue(const GemmArgs& a, int e, int nt, int base, int M,
                                                const float (&res)[NW][KPER]) {
#pragma unroll
  for (int c = 0; c < KPER; ++c) {
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

template <int MT, int NW, int DEPTH>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 2 : 1, MT == 1 ? 2 : 1)))
gemm_decode_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = blockIdx.x, e = blockIdx.y, ks = blockIdx.z;
  const int base = a.offsets[e];
  const int M = a.offsets[e + 1] - base;
  if (M == 0 || M > a.dec_max_rows) return;

  DecodeCtx<MT, NW> cx;
  cx.lane = lane;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    cx.xok[mt] = m < M;
    int xr = 0;
    if (cx.xok[mt]) xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
    cx.xp[mt] = a.x + (size_t)xr * a.K + 8 * (lane >> 4);
  }
#pragma unroll
  for (int f = 0; f < NW; ++f) {
    cx.tbase[f] = a.packed[f] + e * a.words_per_expert + (size_t)nt * a.kblocks * kTileWords;
    cx.sbase[f] = a.sz[f] + e * a.sz_per_expert + (size_t)nt * a.kblocks * kTileSzWords;
  }

  f32x4 acc[NW][MT][4];
#pragma unroll
  for (int f = 0; f < NW; ++f)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K range of this block and the K blocks of this wave: kbw + 4 j, j < cnt
  const int kbA = (int)((int64_t)a.kblocks * ks / a.ksplit);
  const int kbB = (int)((int64_t)a.kblocks * (ks + 1) / a.ksplit);
  const int kb0 = kbA + wave;
  const int kb1 = kbB;
  const int cnt = kb0 < kb1 ? (kb1 - kb0 + 3) / 4 : 0;

  // group sums of the block's rows over its K range -> LDS
  extern __shared__ __align__(16) float smem[];
  const int ngr = 2 * (kbB - kbA);
  cx.lds_xs = smem;
  cx.lds_half = ngr * 16 * MT;
  cx.g0 = 2 * kbA;
  for (int o = threadIdx.x; o < ngr * 16 * MT; o += 256) {
    const int gl = o / (16 * MT), m = o - gl * (16 * MT);
    const size_t src = ((size_t)e * a.groups + cx.g0 + gl) * kDecodeMaxRows + m;
    smem[o] = a.xsum[src];
    smem[cx.lds_half + o] = a.xoff[src];
  }
  __syncthreads();

  Stage<MT, NW> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d)
    if (d < cnt) cx.load(ring[d], kb0 + 4 * d);
  int j = 0;
  // K block of ring entry consumed at step (j + d): kb0 + 4 (j + d)
  // steady state: every prefetch in range, so loads are unconditional and
  // each consume waits only for the batch issued DEPTH-1 steps earlier
  for (; j + 2 * DEPTH - 1 <= cnt; j += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      cx.load(ring[(d + DEPTH - 1) % DEPTH], kb0 + 4 * (j + d + DEPTH - 1));
      cx.consume(ring[d], kb0 + 4 * (j + d), acc);
    }
  }
  // tail: at most 2 DEPTH - 2 blocks left
#pragma unroll
  for (int t = 0; t < 2; ++t, j += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int jn = j + d + DEPTH - 1;
      if (jn < cnt) cx.load(ring[(d + DEPTH - 1) % DEPTH], kb0 + 4 * jn);
      if (j + d < cnt) cx.consume(ring[d], kb0 + 4 * (j + d), acc);
    }
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
  float (*red)[kOut] = (float (*)[kOut])smem;   // reuses the group-sum LDS
  float res[NW][kPer];
#pragma unroll
  for (int f = 0; f < NW; ++f) {
    __syncthreads();
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

  if (a.ksplit > 1) {  // partial sums for gemm_decode_reduce
    float* mine = a.part + (((size_t)ks * a.num_experts + e) * a.n_tiles + nt) * (NW * kOut);
#pragma unroll
    for (int f = 0; f < NW; ++f)
#pragma unroll
      for (int c = 0; c < kPer; ++c) mine[f * kOut + threadIdx.x + 256 * c] = res[f][c];
    return;
  }
  decode_epilogue<NW, kPer>(a, e, nt, base, M, res);
}

// Sum of the K splits in split order, then the epilogue.
template <int MT, int NW>
__global__ void __launch_bounds__(256) gemm_decode_reduce(GemmArgs a) {
  const int nt = blockIdx.x, e = blockIdx.y;
  const int base = a.offsets[e];
  const int M = a.offsets[e + 1] - base;
  if (M == 0 || M > a.dec_max_rows) return;
  constexpr int kOut = MT * 16 * 64;
  constexpr int kPer = kOut / 256;
  float res[NW][kPer];
#pragma unroll
  for (int f = 0; f < NW; ++f)
#pragma unroll
    for (int c = 0; c < kPer; ++c) res[f][c] = 0.f;
  for (int s = 0; s < a.ksplit; ++s) {
    const float* p = a.part + (((size_t)s * a.num_experts + e) * a.n_tiles + nt) * (NW * kOut);
#pragma unroll
    for (int f = 0; f < NW; ++f)
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        const int o = threadIdx.x + 256 * c;
        if ((o >> 6) < M) res[f][c] += p[f * kOut + o];
      }
  }
  decode_epilogue<NW, kPer>(a, e, nt, base, M, res);
}

template <int MT, int NW>
static void launch_mt(const GemmArgs& a, dim3 grid, hipStream_t st) {
  constexpr int depth = (MT == 1 && NW == 1) ? 3 : 2;
  const int max_kb = (a.kblocks + a.ksplit - 1) / a.ksplit + 1;
  size_t lds = (size_t)2 * 2 * max_kb * 16 * MT * sizeof(float);
  const size_t red = (size_t)4 * MT * 16 * 64 * sizeof(float);
  if (lds < red) lds = red;
  hipLaunchKernelGGL((gemm_decode_kernel<MT, NW, depth>), grid, dim3(256), lds, st, a);
  if (a.ksplit > 1)
    hipLaunchKernelGGL((gemm_decode_reduce<MT, NW>), dim3(grid.x, grid.y), dim3(256), 0, st, a);
}

GemmArgs make_gemm_args(const milo_gemm_desc* d, const GemmPlan& p, char* ws);

int32_t launch_gemm_decode(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  if (p.dec_mt == 0) return MILO_OK;
  GemmArgs a = make_gemm_args(d, p, ws);
  a.part = (float*)(ws + p.off_dec_part);
  dim3 grid(p.n_tiles, d->num_experts, p.dec_ksplit);
  const bool two = d->n_w == 2;
  switch (p.dec_mt) {
    case 1: two ? launch_mt<1, 2>(a, grid, st) : launch_mt<1, 1>(a, grid, st); break;
    case 2: two ? launch_mt<2, 2>(a, grid, st) : launch_mt<2, 1>(a, grid, st); break;
    default: set_error("internal: bad m-tile count %d", p.dec_mt); return MILO_ERR_ARG;
  }
  return hip_status(hipGetLastError(), "gemm_decode_kernel launch");
}

}  // namespace milo
