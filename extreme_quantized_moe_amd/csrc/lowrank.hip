// Low-rank pre-pass of the compensated GEMM: T = x_rows(e) . V_e^T per pair.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), MiLo Algorithm: the weight is
// W_quant + U V (U out x R, V R x in), so x . W^T = x . deq(W)^T + (x . V^T) . U^T.
// The product x . V^T depends only on the pair's row and its expert, not on the
// output tile, so it is computed once per pair here (fp32 accumulation on the
// matrix cores) and stored as float16 for the GEMM kernels, which add
// T . U^T as two more matrix-core K-steps.
//
// Grid: x = 16-row tiles over all experts (expert by expert), y = K chunks.
// The four waves of a block split the chunk's 32-wide K steps round robin and
// are summed in LDS in wave order; K chunks are summed by the last block of a
// tile to finish, in chunk order (deterministic).
#include "milo_internal.hpp"

namespace milo {

struct LowrankArgs {
  const uint16_t* x;
  const int32_t* sorted_pairs;
  const int32_t* offsets;
  const uint16_t* V[2];
  const int32_t* rank[2];
  uint16_t* T;        // fp16 [P][n_w * rp]
  float* part;        // fp32 [kchunks][tiles][16][n_w * rp]
  int32_t* cnt;       // [tiles]
  int K, gather_div, num_experts, n_w, rp, max_rank, kchunks;
};

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

template <int NRT>  // rank tiles of 16 columns (n_w * rp / 16)
__global__ void __launch_bounds__(256) lowrank_kernel(LowrankArgs a) {
  __shared__ float red[4][NRT][64][4];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e, m0, M;
  if (!find_tile16(a.offsets, a.num_experts, blockIdx.x, &e, &m0, &M)) return;
  const int base = a.offsets[e];
  const int RW = a.n_w * a.rp;
  const int tiles_per_w = a.rp / 16;

  // A operand row of this lane
  const int m = m0 + (lane & 15);
  const bool row_ok = m < M;
  int xr = 0;
  if (row_ok) xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
  const uint16_t* xp = a.x + (size_t)xr * a.K + 8 * (lane >> 4);

  // B operand rows (compensator ranks) of this lane, per rank tile
  const uint16_t* vp[NRT];
  bool vok[NRT];
#pragma unroll
  for (int tr = 0; tr < NRT; ++tr) {
    const int f = tr / tiles_per_w;
    const int j = (tr % tiles_per_w) * 16 + (lane & 15);
    vok[tr] = j < a.rank[f][e];
    vp[tr] = a.V[f] + ((size_t)e * a.max_rank + (vok[tr] ? j : 0)) * a.K + 8 * (lane >> 4);
  }

  f32x4 acc[NRT];
#pragma unroll
  for (int tr = 0; tr < NRT; ++tr) acc[tr] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = a.K / 32;
  const int s0 = (int)((int64_t)ksteps * blockIdx.y / a.kchunks);
  const int s1 = (int)((int64_t)ksteps * (blockIdx.y + 1) / a.kchunks);
  for (int s = s0 + wave; s < s1; s += 4) {
    f16x8 xa = f16x8{};
    if (row_ok) xa = *(const f16x8*)(xp + 32 * s);
#pragma unroll
    for (int tr = 0; tr < NRT; ++tr) {
      f16x8 vb = f16x8{};
      if (vok[tr]) vb = *(const f16x8*)(vp[tr] + 32 * s);
      acc[tr] = mfma16x16x32(xa, vb, acc[tr]);
    }
  }
#pragma unroll
  for (int tr = 0; tr < NRT; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][tr][lane][r] = acc[tr][r];
  __syncthreads();

  // thread -> (rank tile, lane, r) outputs: NRT * 256 values over 256 threads
  for (int o = threadIdx.x; o < NRT * 256; o += 256) {
    const int tr = o >> 8, ln = (o >> 2) & 63, r = o & 3;
    const float v = red[0][tr][ln][r] + red[1][tr][ln][r] + red[2][tr][ln][r] + red[3][tr][ln][r];
    const int row = 4 * (ln >> 4) + r;            // 0..15 within the tile
    const int col = tr * 16 + (ln & 15);          // 0..RW-1
    if (a.kchunks == 1) {
      if (m0 + row < M) a.T[(size_t)(base + m0 + row) * RW + col] = float_to_half_bits(v);
    } else {
      a.part[(((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 16 + row) * RW + col] = v;
    }
  }
  if (a.kchunks == 1) return;

  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&a.cnt[blockIdx.x], 1);
    is_last = (prev == a.kchunks - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int o = threadIdx.x; o < 16 * RW; o += 256) {
    const int row = o / RW, col = o - row * RW;
    float v = 0.f;
    for (int c = 0; c < a.kchunks; ++c)
      v += __builtin_nontemporal_load(&a.part[(((size_t)c * gridDim.x + blockIdx.x) * 16 + row) * RW + col]);
    if (m0 + row < M) a.T[(size_t)(base + m0 + row) * RW + col] = float_to_half_bits(v);
  }
  if (threadIdx.x == 0) a.cnt[blockIdx.x] = 0;
}

int32_t launch_lowrank(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  if (p.rp == 0) return MILO_OK;
  LowrankArgs a;
  a.x = d->x;
  a.sorted_pairs = d->sorted_pairs;
  a.offsets = d->offsets;
  for (int f = 0; f < 2; ++f) {
    a.V[f] = d->w[f < d->n_w ? f : 0].V;
    a.rank[f] = d->w[f < d->n_w ? f : 0].rank;
  }
  a.T = (uint16_t*)(ws + p.off_t);
  a.part = (float*)(ws + p.off_lr_part);
  a.cnt = (int32_t*)(ws + p.off_lr_cnt);
  a.K = d->K;
  a.gather_div = d->gather_div;
  a.num_experts = d->num_experts;
  a.n_w = d->n_w;
  a.rp = p.rp;
  a.max_rank = d->max_rank;
  a.kchunks = p.lr_kchunks;
  const int nrt = d->n_w * p.rp / 16;
  dim3 grid(p.lr_tiles, p.lr_kchunks);
  switch (nrt) {
    case 2: hipLaunchKernelGGL(lowrank_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(lowrank_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(lowrank_kernel<8>, grid, dim3(256), 0, st, a); break;
    default:
      set_error("internal: unsupported rank-tile count %d", nrt);
      return MILO_ERR_RANK;
  }
  return hip_status(hipGetLastError(), "lowrank_kernel launch");
}

}  // namespace milo
