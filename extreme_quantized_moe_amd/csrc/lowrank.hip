// Pre-pass of the compensated GEMM: the low-rank products T = x_rows(e) . V_e^T
// per pair, and (for the small-M kernel) the pair-ordered copy of the gathered
// activation rows and the per-pair route weights.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), MiLo Algorithm: the weight is
// W_quant + U V (U out x R, V R x in), so x . W^T = x . deq(W)^T + (x . V^T) . U^T.
// The product x . V^T depends only on the pair's row and its expert, not on the
// output tile, so it is computed once per pair here (fp32 accumulation on the
// matrix cores) and stored as float16 for the GEMM kernels, which add
// T . U^T as two more matrix-core K-steps.
//
// Grid: x = 16-row tiles over all experts (expert by expert); y = compensator
// ranks (decode) or groups of NRT rank tiles of 16 ranks (prefill), plus one
// "aux" index for the gather / pair weights.
// At decode (at most 32 rows per expert) a block computes one rank j of T for
// its rows as plain dot products: the 256 threads read V row j in consecutive
// 16-byte chunks (fully coalesced) and multiply with the same chunks of each
// row; the per-thread partial sums are added in LDS in a fixed tree order.
// At prefill a block is 4 waves on every rank tile of its rows on the matrix
// cores (the activation rows are read once); wave partial sums are added in
// LDS in wave order.
#include "milo_internal.hpp"

namespace milo {

struct PrepassArgs {
  const uint16_t* x;
  const int32_t* sorted_pairs;
  const int32_t* offsets;
  const float* slot_w;
  const uint16_t* V[2];
  const int32_t* rank[2];
  uint16_t* T;        // fp16 [P][n_w * rp]
  uint16_t* xg;       // fp16 [P][K]: row of each pair (small-M experts), or null
  float* pw;          // fp32 [P]: route weight of each pair, or null
  int K, gather_div, num_experts, n_w, rp, max_rank;
  int aux_y;          // blockIdx.y of the aux blocks (-1: none)
  int dec_max_rows;   // experts with more rows are not gathered
};

__device__ __forceinline__ bool find_tile16(const int32_t* offsets, int num_experts, int tile,
                                            int* e_out, int* m0_out, int* rows_out) {
  return find_row_tile(offsets, num_experts, 0, 16, tile, e_out, m0_out, rows_out);
}

// Gathered rows (pair order) and pair weights of one 16-row tile.
__device__ void prepass_aux(const PrepassArgs& a, int e, int m0, int M) {
  const int base = a.offsets[e];
  const int rows = (M - m0) < 16 ? (M - m0) : 16;
  if (a.pw && threadIdx.x < rows) {
    const int i = base + m0 + threadIdx.x;
    a.pw[i] = a.slot_w[a.sorted_pairs[i]];
  }
  if (!a.xg || M > a.dec_max_rows) return;
  // copy the tile's rows in pair order, eight 16-byte chunks in flight per thread
  const int chunks = a.K / 8;                     // 16-byte chunks per row
  const int n = rows * chunks;
  for (int o0 = threadIdx.x; o0 < n; o0 += 8 * blockDim.x) {
    u32x4 v[8];
    size_t dst[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = o0 + u * blockDim.x;
      dst[u] = 0;
      if (o < n) {
        const int r = o / chunks, c = o - r * chunks;
        const int i = base + m0 + r;
        const int xr = a.sorted_pairs[i] / a.gather_div;
        v[u] = *(const u32x4*)(a.x + (size_t)xr * a.K + 8 * c);
        dst[u] = (size_t)i * a.K + 8 * c;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (o0 + u * blockDim.x < n) *(u32x4*)(a.xg + dst[u]) = v[u];
  }
}

// Decode form: block (16-row tile, rank j over all families), 512 threads.
// The rows of the tile are rounded up to R2 (a power of two) and each row gets
// 512 / R2 consecutive threads, which stride over the 16-byte chunks of V row j
// and of the token row, eight chunks per batch of loads.  The partial sums of a
// row are reduced in a fixed order: a butterfly inside each wave, then the
// waves of that row in ascending order.
constexpr int kDotThreads = 512;
constexpr int kDotBatch = 8;

__global__ void __launch_bounds__(kDotThreads) prepass_dot_kernel(PrepassArgs a) {
  __shared__ float part[kDotThreads / 64];
  int e, m0, M;
  if (!find_tile16(a.offsets, a.num_experts, blockIdx.x, &e, &m0, &M)) return;
  if ((int)blockIdx.y == a.aux_y) {
    prepass_aux(a, e, m0, M);
    return;
  }
  const int base = a.offsets[e];
  const int RW = a.n_w * a.rp;
  const int f = blockIdx.y / a.rp, j = blockIdx.y - f * a.rp;
  const int rows = (M - m0) < 16 ? (M - m0) : 16;
  const int tid = threadIdx.x;
  uint16_t* tout = a.T + (size_t)(base + m0) * RW + f * a.rp + j;
  if (j >= a.rank[f][e]) {                        // beyond the expert's rank: T = 0
    if (tid < rows) tout[(size_t)tid * RW] = 0;
    return;
  }
  const int R2 = rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16;
  const int G = kDotThreads / R2;                 // threads per row, 32 .. 512
  const int r = tid / G, g = tid - r * G;
  const int chunks = a.K / 8;
  float acc = 0.f;
  if (r < rows) {
    const int i = base + m0 + r;
    const int xr = a.gather_div > 0 ? a.sorted_pairs[i] / a.gather_div : i;
    const uint16_t* xp = a.x + (size_t)xr * a.K;
    const uint16_t* vp = a.V[f] + ((size_t)e * a.max_rank + j) * a.K;
    for (int c0 = g; c0 < chunks; c0 += kDotBatch * G) {
      f16x8 v[kDotBatch], xv[kDotBatch];
#pragma unroll
      for (int u = 0; u < kDotBatch; ++u) {
        const int c = c0 + G * u;
        v[u] = c < chunks ? *(const f16x8*)(vp + 8 * c) : f16x8{};
        xv[u] = c < chunks ? *(const f16x8*)(xp + 8 * c) : f16x8{};
      }
#pragma unroll
      for (int u = 0; u < kDotBatch; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = __builtin_fmaf((float)xv[u][t], (float)v[u][t], acc);
    }
  }
  const int W = G < 64 ? G : 64;
  for (int o = W >> 1; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (G < 64) {
    if (g == 0 && r < rows) tout[(size_t)r * RW] = float_to_half_bits(acc);
    return;
  }
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  const int wpr = G >> 6;                         // waves per row
  if (tid < rows) {
    float sum = 0.f;
    for (int w = 0; w < wpr; ++w) sum += part[tid * wpr + w];
    tout[(size_t)tid * RW] = float_to_half_bits(sum);
  }
}

template <int NRT, int NWAVES, int UNR>
__global__ void __launch_bounds__(64 * NWAVES) prepass_kernel(PrepassArgs a) {
  __shared__ float red[NWAVES][NRT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, m0, M;
  if (!find_tile16(a.offsets, a.num_experts, blockIdx.x, &e, &m0, &M)) return;
  if ((int)blockIdx.y == a.aux_y) {
    prepass_aux(a, e, m0, M);
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

  // K steps s = wave + NWAVES i, in batches of UNR steps whose loads are all
  // issued before the first product (steps past the end are skipped)
  const int ksteps = a.K / 32;
  if (any) {
    for (int s0 = wave; s0 < ksteps; s0 += UNR * NWAVES) {
      f16x8 xa[UNR], vb[UNR][NRT];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int s = s0 + NWAVES * u;
        const bool in = s < ksteps;
        xa[u] = (in && row_ok) ? *(const f16x8*)(xp + 32 * s) : f16x8{};
#pragma unroll
        for (int t = 0; t < NRT; ++t)
          vb[u][t] = (in && vok[t]) ? *(const f16x8*)(vp[t] + 32 * s) : f16x8{};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int t = 0; t < NRT; ++t) acc[t] = mfma16x16x32(xa[u], vb[u][t], acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][t][lane][r] = acc[t][r];
  __syncthreads();

  for (int o = threadIdx.x; o < NRT * 256; o += 64 * NWAVES) {
    const int t = o >> 8, ln = (o >> 2) & 63, r = o & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) v += red[w][t][ln][r];
    const int row = 4 * (ln >> 4) + r;            // 0..15 within the tile
    const int col = (tr0 + t) * 16 + (ln & 15);   // 0..RW-1
    if (m0 + row < M) a.T[(size_t)(base + m0 + row) * RW + col] = float_to_half_bits(v);
  }
}

int32_t launch_lowrank(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  const int nrt = d->n_w * p.rp / 16;                   // rank tiles in total
  const int per = p.rp ? p.lr_tiles_per_block : 1;      // 1 (decode) or nrt (prefill)
  const int rank_blocks = p.rp ? nrt / per : 0;
  const bool need_xg = p.dec_mt && d->gather_div > 0;
  const bool need_pw = p.dec_mt && d->epilogue == MILO_EPI_ROUTE_SCALE;
  const int aux_blocks = (need_xg || need_pw) ? 1 : 0;
  if (rank_blocks + aux_blocks == 0) return MILO_OK;
  PrepassArgs a;
  a.x = d->x;
  a.sorted_pairs = d->sorted_pairs;
  a.offsets = d->offsets;
  a.slot_w = d->slot_w;
  for (int f = 0; f < 2; ++f) {
    a.V[f] = d->w[f < d->n_w ? f : 0].V;
    a.rank[f] = d->w[f < d->n_w ? f : 0].rank;
  }
  a.T = (uint16_t*)(ws + p.off_t);
  a.xg = need_xg ? (uint16_t*)(ws + p.off_xg) : nullptr;
  a.pw = need_pw ? (float*)(ws + p.off_pw) : nullptr;
  a.K = d->K;
  a.gather_div = d->gather_div;
  a.num_experts = d->num_experts;
  a.n_w = d->n_w;
  a.rp = p.rp;
  a.max_rank = d->max_rank;
  a.aux_y = aux_blocks ? rank_blocks : -1;
  a.dec_max_rows = p.dec_max_rows;
  if (per == 1) {                                   // decode: one block per rank
    const int rank_rows = p.rp ? d->n_w * p.rp : 0;
    a.aux_y = aux_blocks ? rank_rows : -1;
    dim3 grid(p.lr_tiles, rank_rows + aux_blocks);
    hipLaunchKernelGGL(prepass_dot_kernel, grid, dim3(kDotThreads), 0, st, a);
  } else {
    dim3 grid(p.lr_tiles, rank_blocks + aux_blocks);
    switch (per) {
      case 2: hipLaunchKernelGGL((prepass_kernel<2, 4, 4>), grid, dim3(256), 0, st, a); break;
      case 4: hipLaunchKernelGGL((prepass_kernel<4, 4, 4>), grid, dim3(256), 0, st, a); break;
      case 8: hipLaunchKernelGGL((prepass_kernel<8, 4, 4>), grid, dim3(256), 0, st, a); break;
      default:
        set_error("internal: unsupported rank-tile count %d", per);
        return MILO_ERR_RANK;
    }
  }
  return hip_status(hipGetLastError(), "prepass_kernel launch");
}

}  // namespace milo
