// Low-rank pre-pass of the compensated GEMM: T = x_rows(e) . V_e^T per pair,
// plus the per-(row, group) activation sums the small-M kernel folds with.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), MiLo Algorithm: the weight is
// W_quant + U V (U out x R, V R x in), so x . W^T = x . deq(W)^T + (x . V^T) . U^T.
// The product x . V^T depends only on the pair's row and its expert, not on the
// output tile, so it is computed once per pair here (fp32 accumulation on the
// matrix cores) and stored as float16 for the GEMM kernels, which add
// T . U^T as two more matrix-core K-steps.
//
// Grid: x = 16-row tiles over all experts (expert by expert), y = groups of
// NRT rank tiles (16 ranks each) plus, when the small-M kernel runs, one more
// index for the group sums, z = K chunks.  At decode each block takes one rank
// tile of one K chunk (many small blocks stream V in parallel); at prefill one
// block takes every rank tile of its rows over the whole K (the activation
// rows are read once).  The four waves of a block split the chunk's 32-wide K
// steps round robin and are added in LDS in wave order.  With several K chunks
// the chunk sums go to a float32 buffer and lowrank_finalize adds them in
// chunk order (deterministic; no cross-block synchronisation in a kernel).
#include "milo_internal.hpp"

namespace milo {

struct LowrankArgs {
  const uint16_t* x;
  const int32_t* sorted_pairs;
  const int32_t* offsets;
  const uint16_t* V[2];
  const int32_t* rank[2];
  uint16_t* T;        // fp16 [P][n_w * rp]
  float* part;        // fp32 [kchunks][P][n_w * rp] when kchunks > 1
  float* xsum;        // [expert][group][32 rows]: sum of x over the group
  float* xoff;        // [expert][group][32 rows]: sum of x * off over the group
  int K, gather_div, num_experts, n_w, rp, max_rank, num_pairs;
  int xs_y;           // blockIdx.y of the group-sum blocks (-1: none)
  int dec_max_rows;   // experts with more rows need no group sums
  int kchunks;
};

// Offset (64 or 8) of the "off + q" float16 encoding of the code at position
// kk (0..127) of a 128-wide K block: code c = 8 (kk div 32) + kk mod 8 of the
// lane's triplet, pair c div 2.
__device__ __forceinline__ float code_offset(int kk) {
  const int c = 8 * (kk >> 5) + (kk & 7);
  return (float)pair_offset(c >> 1);
}

// Per (row, 64-wide group) of this block's K chunk: sum of x and sum of
// x * off, each in a fixed order.
__device__ void group_sums(const LowrankArgs& a, int e, int m0, int M) {
  if (M > a.dec_max_rows) return;                 // tile-kernel expert
  const int base = a.offsets[e];
  const int G = a.K / kGroup;
  const int g0 = (int)((int64_t)G * blockIdx.z / a.kchunks);
  const int g1 = (int)((int64_t)G * (blockIdx.z + 1) / a.kchunks);
  const int ng = g1 - g0;
  for (int o = threadIdx.x; o < 16 * ng; o += blockDim.x) {
    const int row = o / ng, g = g0 + (o - row * ng);
    const int m = m0 + row;
    if (m >= M) continue;
    const int xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
    const uint16_t* p = a.x + (size_t)xr * a.K + (size_t)g * kGroup;
    f16x8 v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = *(const f16x8*)(p + 8 * c);
    float sx = 0.f, so = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xv = (float)v[c][t];
        sx += xv;
        so = __builtin_fmaf(xv, code_offset(64 * (g & 1) + 8 * c + t), so);
      }
    const size_t oi = ((size_t)e * G + g) * kDecodeMaxRows + m;
    a.xsum[oi] = sx;
    a.xoff[oi] = so;
  }
}

// Locate the (expert, first row) of 16-row tile `tile`; returns false past the end.
__device__ __forceinline__ bool find_tile16(const int32_t* offsets, int num_experts, int tile,
                                            int* e_out, int* m0_out, int* rows_out) {
  int cum = 0;
  for (int e = 0; e < num_experts; ++e) {
    const int m = offsets[e + 1] - offsets[e];
    const int nt = (m + 15) >> 4;
    if (tile < cum + nt) {
      *e_out = e;
      *m0_out = (tile - cum) * 16;
      *rows_out = m;
      return true;
    }
    cum += nt;
  }
  return false;
}

template <int NRT>  // rank tiles of 16 columns per block
__global__ void __launch_bounds__(256) lowrank_kernel(LowrankArgs a) {
  __shared__ float red[4][NRT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, m0, M;
  if (!find_tile16(a.offsets, a.num_experts, blockIdx.x, &e, &m0, &M)) return;
  if ((int)blockIdx.y == a.xs_y) {
    group_sums(a, e, m0, M);
    return;
  }
  const int base = a.offsets[e];
  const int RW = a.n_w * a.rp;
  const int tiles_per_w = a.rp / 16;
  const int tr0 = blockIdx.y * NRT;            // first rank tile of this block

  // A operand row of this lane
  const int m = m0 + (lane & 15);
  const bool row_ok = m < M;
  int xr = 0;
  if (row_ok) xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
  const uint16_t* xp = a.x + (size_t)xr * a.K + 8 * (lane >> 4);

  // B operand rows (compensator ranks) of this lane, per rank tile
  const uint16_t* vp[NRT];
  bool vok[NRT];
  bool any = false;
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const int tr = tr0 + t;
    const int f = tr / tiles_per_w;
    const int j = (tr % tiles_per_w) * 16 + (lane & 15);
    vok[t] = j < a.rank[f][e];
    any |= (tr % tiles_per_w) * 16 < a.rank[f][e];
    vp[t] = a.V[f] + ((size_t)e * a.max_rank + (vok[t] ? j : 0)) * a.K + 8 * (lane >> 4);
  }

  f32x4 acc[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this block's K steps [s0, s1); wave takes s0 + wave + 4 i, loads batched by 4
  const int ksteps = a.K / 32;
  const int s0 = (int)((int64_t)ksteps * blockIdx.z / a.kchunks);
  const int s1 = (int)((int64_t)ksteps * (blockIdx.z + 1) / a.kchunks);
  if (any) {
    int s = s0 + wave;
    for (; s + 12 < s1; s += 16) {
      f16x8 xa[4], vb[4][NRT];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xa[u] = row_ok ? *(const f16x8*)(xp + 32 * (s + 4 * u)) : f16x8{};
#pragma unroll
        for (int t = 0; t < NRT; ++t)
          vb[u][t] = vok[t] ? *(const f16x8*)(vp[t] + 32 * (s + 4 * u)) : f16x8{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < NRT; ++t) acc[t] = mfma16x16x32(xa[u], vb[u][t], acc[t]);
    }
    for (; s < s1; s += 4) {
      const f16x8 xa = row_ok ? *(const f16x8*)(xp + 32 * s) : f16x8{};
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
        const f16x8 vb = vok[t] ? *(const f16x8*)(vp[t] + 32 * s) : f16x8{};
        acc[t] = mfma16x16x32(xa, vb, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][t][lane][r] = acc[t][r];
  __syncthreads();

  for (int o = threadIdx.x; o < NRT * 256; o += 256) {
    const int t = o >> 8, ln = (o >> 2) & 63, r = o & 3;
    const float v = ((red[0][t][ln][r] + red[1][t][ln][r]) + red[2][t][ln][r]) + red[3][t][ln][r];
    const int row = 4 * (ln >> 4) + r;            // 0..15 within the tile
    const int col = (tr0 + t) * 16 + (ln & 15);   // 0..RW-1
    if (m0 + row >= M) continue;
    const size_t i = (size_t)(base + m0 + row) * RW + col;
    if (a.kchunks == 1)
      a.T[i] = float_to_half_bits(v);
    else
      a.part[(size_t)blockIdx.z * a.num_pairs * RW + i] = v;
  }
}

// T = fp16(sum of the K-chunk partial products, in chunk order)
__global__ void __launch_bounds__(256) lowrank_finalize(const float* __restrict__ part, int kchunks,
                                                        size_t n, uint16_t* __restrict__ T) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    for (int c = 0; c < kchunks; ++c) v += part[(size_t)c * n + i];
    T[i] = float_to_half_bits(v);
  }
}

int32_t launch_lowrank(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  const int nrt = d->n_w * p.rp / 16;                   // rank tiles in total
  const int per = p.rp ? p.lr_tiles_per_block : 1;      // 1 (decode) or nrt (prefill)
  const int rank_blocks = p.rp ? nrt / per : 0;
  const int xs_blocks = p.dec_mt ? 1 : 0;
  if (rank_blocks + xs_blocks == 0) return MILO_OK;
  LowrankArgs a;
  a.x = d->x;
  a.sorted_pairs = d->sorted_pairs;
  a.offsets = d->offsets;
  for (int f = 0; f < 2; ++f) {
    a.V[f] = d->w[f < d->n_w ? f : 0].V;
    a.rank[f] = d->w[f < d->n_w ? f : 0].rank;
  }
  a.T = (uint16_t*)(ws + p.off_t);
  a.part = (float*)(ws + p.off_tpart);
  a.xsum = (float*)(ws + p.off_xs);
  a.xoff = a.xsum + (size_t)d->num_experts * (d->K / kGroup) * kDecodeMaxRows;
  a.K = d->K;
  a.gather_div = d->gather_div;
  a.num_experts = d->num_experts;
  a.n_w = d->n_w;
  a.rp = p.rp;
  a.max_rank = d->max_rank;
  a.num_pairs = d->num_pairs;
  a.xs_y = xs_blocks ? rank_blocks : -1;
  a.dec_max_rows = p.dec_max_rows;
  a.kchunks = p.lr_kchunks;
  dim3 grid(p.lr_tiles, rank_blocks + xs_blocks, p.lr_kchunks);
  switch (per) {
    case 1: hipLaunchKernelGGL(lowrank_kernel<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(lowrank_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(lowrank_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(lowrank_kernel<8>, grid, dim3(256), 0, st, a); break;
    default:
      set_error("internal: unsupported rank-tile count %d", per);
      return MILO_ERR_RANK;
  }
  int32_t rc = hip_status(hipGetLastError(), "lowrank_kernel launch");
  if (rc != MILO_OK || p.lr_kchunks == 1 || p.rp == 0) return rc;
  const size_t n = (size_t)d->num_pairs * d->n_w * p.rp;
  size_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(lowrank_finalize, dim3((unsigned)g), dim3(256), 0, st, (const float*)a.part,
                     p.lr_kchunks, n, a.T);
  return hip_status(hipGetLastError(), "lowrank_finalize launch");
}

}  // namespace milo
