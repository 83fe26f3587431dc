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
// Grid: x = row tiles over all experts (expert by expert); y = compensator
// ranks or groups of them (decode) or groups of rank tiles of 16 ranks
// (prefill), plus one "aux" index for the gather / pair weights; z = K chunks
// (prefill forms, fp16 V) when the rows alone give a sparse grid.
// At decode (at most 32 rows per expert) a block computes one rank (fp16 V)
// or four ranks (int3 V) of T for its rows as plain dot products over
// coalesced chunks of the V rows and the activation rows; per-thread partial
// sums are added in a fixed tree order.  At prefill the products run on the
// matrix cores: 128-row tiles with every rank tile per block where experts
// average 128 rows or more, else 16-row tiles x groups of rank tiles with
// wave partial sums added in LDS in wave order; K-chunk partials (fp32) are
// added in chunk order by a reduce pass.  int3 factors ([talk] MiLo
// Algorithm, last step: U and V stored as int3) are dequantized in
// registers: folded into the dot products at decode, to fp16 matrix-core
// operands at prefill.
#include "gemm_common.hpp"

namespace milo {

struct PrepassArgs {
  const uint16_t* x;
  const int32_t* sorted_pairs;
  const int32_t* offsets;
  const float* slot_w;
  const uint16_t* V[2];
  const uint32_t* Vq[2];    // int3 factors: V layout codes and scale/zero
  const uint32_t* Vsz[2];
  int64_t vq_per_expert, vsz_per_expert;
  const int32_t* rank[2];
  uint16_t* T;        // fp16 [P][n_w * rp]
  float* tpart;       // fp32 [ks][P][n_w * rp]: K-chunk partials of T (prefill form, ks > 1), or null
  int ks_steps;       // 32-wide K steps per chunk (prefill form)
  int num_pairs;
  uint16_t* xg;       // fp16 [P][K]: row of each pair (small-M experts), or null
  float* pw;          // fp32 [P]: route weight of each pair, or null
  int K, gather_div, num_experts, n_w, rp, max_rank;
  int aux_y;          // first blockIdx.y of the aux blocks (-1: none)
  int aux_parts;      // aux blocks per row tile along y (each copies a share of the rows)
  int dec_max_rows;   // experts with more rows are not gathered
};

// The block's 16-row tile (all experts with rows), with the expert's first
// pair and its ranks in both families.
__device__ __forceinline__ bool find_tile16(const PrepassArgs& a, RowTile* t) {
  return find_row_tile(a.offsets, a.num_experts, 0, 16, blockIdx.x, a.rp ? a.rank[0] : nullptr,
                       a.rp ? a.rank[1] : nullptr, t);
}

// Gathered rows (pair order) and pair weights of one 16-row tile; part
// `part` of `parts` of the rows' 16-byte chunks (the weights with part 0).
__device__ void prepass_aux(const PrepassArgs& a, int base, int m0, int M, int part = 0, int parts = 1) {
  const int rows = (M - m0) < 16 ? (M - m0) : 16;
  if (a.pw && part == 0 && (int)threadIdx.x < rows) {
    const int i = base + m0 + threadIdx.x;
    a.pw[i] = a.slot_w[a.sorted_pairs[i]];
  }
  if (!a.xg || M > a.dec_max_rows) return;
  // copy the tile's rows in pair order, eight 16-byte chunks in flight per thread
  const int chunks = a.K / 8;                     // 16-byte chunks per row
  const int n = rows * chunks;
  const int o_end = (int)((int64_t)n * (part + 1) / parts);
  for (int o0 = (int)((int64_t)n * part / parts) + threadIdx.x; o0 < o_end; o0 += 8 * blockDim.x) {
    u32x4 v[8];
    size_t dst[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = o0 + u * blockDim.x;
      dst[u] = 0;
      if (o < o_end) {
        const int r = o / chunks, c = o - r * chunks;
        const int i = base + m0 + r;
        const int xr = a.sorted_pairs[i] / a.gather_div;
        v[u] = *(const u32x4*)(a.x + (size_t)xr * a.K + 8 * c);
        dst[u] = (size_t)i * a.K + 8 * c;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (o0 + u * (int)blockDim.x < o_end) *(u32x4*)(a.xg + dst[u]) = v[u];
  }
}

// Aux block test and share for the grid.y layout [rank blocks | aux_parts].
__device__ __forceinline__ bool is_aux(const PrepassArgs& a) {
  return a.aux_y >= 0 && (int)blockIdx.y >= a.aux_y;
}

constexpr int kDotThreads = 512;

// Decode form, fp16 V: block (16-row tile, rank j over all families), THREADS
// threads (256 for K <= 4096: the grid then fits the GPU in one round; 512
// above, for more loads in flight per row).
// The rows of the tile are rounded up to R2 (a power of two) and each row gets
// THREADS / R2 consecutive threads, which stride over the 16-byte chunks of V row j
// and of the token row, eight chunks per batch of loads.  The partial sums of a
// row are reduced in a fixed order: a butterfly inside each wave, then the
// waves of that row in ascending order.
constexpr int kDotBatch = 8;

template <int THREADS>
__global__ void __launch_bounds__(THREADS) prepass_dot_kernel(PrepassArgs a) {
  __shared__ float part[THREADS / 64];
  RowTile rt;
  if (!find_tile16(a, &rt)) return;
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  if (is_aux(a)) {
    prepass_aux(a, base, m0, M, blockIdx.y - a.aux_y, a.aux_parts);
    return;
  }
  const int RW = a.n_w * a.rp;
  const int f = blockIdx.y / a.rp, j = blockIdx.y - f * a.rp;
  const int rows = (M - m0) < 16 ? (M - m0) : 16;
  const int tid = threadIdx.x;
  uint16_t* tout = a.T + (size_t)(base + m0) * RW + f * a.rp + j;
  if (j >= rt.rank(f)) {                          // beyond the expert's rank: T = 0
    if (tid < rows) tout[(size_t)tid * RW] = 0;
    return;
  }
  const int R2 = rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16;
  const int G = THREADS / R2;                     // threads per row, 16 .. THREADS
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

// Decode form, int3 V: block = (16-row tile, NJ consecutive ranks of one family),
// 512 threads.  The rows of the tile are rounded up to R2 (a power of two) and
// each row gets 512 / R2 consecutive threads, which stride over the row's K
// (16-byte chunks of fp16 V, or 32-column triplets of int3 V), reading each
// activation chunk once for the NJ ranks.  The partial sums of a (row, rank)
// are reduced in a fixed order: a butterfly inside each wave, then the waves
// of that row in ascending order.  Ranks at or beyond the expert's rank give
// T = 0 (their V rows are not read).

template <int NJ>
__device__ __forceinline__ void dot_reduce_store(float (&acc)[NJ], int G, int rows, uint16_t* tout,
                                                 int RW, float* part) {
  const int tid = threadIdx.x, r = tid / G, g = tid - r * G;
  const int W = G < 64 ? G : 64;
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
    for (int o = W >> 1; o >= 1; o >>= 1) acc[jj] += __shfl_xor(acc[jj], o);
  if (G < 64) {
    if (g == 0 && r < rows)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) tout[(size_t)r * RW + jj] = float_to_half_bits(acc[jj]);
    return;
  }
  if ((tid & 63) == 0)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) part[jj * (kDotThreads / 64) + (tid >> 6)] = acc[jj];
  __syncthreads();
  const int wpr = G >> 6;                         // waves per row
  if (tid < rows * NJ) {
    const int rr = tid / NJ, jj = tid - rr * NJ;
    float sum = 0.f;
    for (int w = 0; w < wpr; ++w) sum += part[jj * (kDotThreads / 64) + rr * wpr + w];
    tout[(size_t)rr * RW + jj] = float_to_half_bits(sum);
  }
}

// Common prologue of the decode forms: tile lookup, aux blocks, and the
// block's (family, first rank, rows).  Returns false if the block is done.
struct DotBlock {
  int e, m0, M, base, RW, f, j0, rk, rows, R2, G, r, g;
  uint16_t* tout;
};

template <int NJ>
__device__ __forceinline__ bool dot_block(const PrepassArgs& a, DotBlock& b) {
  RowTile rt;
  if (!find_tile16(a, &rt)) return false;
  b.e = rt.e;
  b.m0 = rt.m0;
  b.M = rt.rows;
  b.base = rt.base;
  if (is_aux(a)) {
    prepass_aux(a, b.base, b.m0, b.M, blockIdx.y - a.aux_y, a.aux_parts);
    return false;
  }
  b.RW = a.n_w * a.rp;
  const int y0 = blockIdx.y * NJ;
  b.f = y0 / a.rp;
  b.j0 = y0 - b.f * a.rp;
  b.rows = (b.M - b.m0) < 16 ? (b.M - b.m0) : 16;
  b.tout = a.T + (size_t)(b.base + b.m0) * b.RW + b.f * a.rp + b.j0;
  b.rk = rt.rank(b.f);
  const int tid = threadIdx.x;
  if (b.j0 >= b.rk) {                             // beyond the expert's rank: T = 0
    if (tid < b.rows * NJ) b.tout[(size_t)(tid / NJ) * b.RW + tid % NJ] = 0;
    return false;
  }
  b.R2 = b.rows <= 1 ? 1 : b.rows <= 2 ? 2 : b.rows <= 4 ? 4 : b.rows <= 8 ? 8 : 16;
  b.G = kDotThreads / b.R2;                       // threads per row, 32 .. 512
  b.r = tid / b.G;
  b.g = tid - b.r * b.G;
  return true;
}

// int3 V (row layout): triplets of 32 columns, two per batch of loads.
// Dequantization is folded out of the dot product: v_dot2 forms
// sum x (off + q) per 64-wide group from the extracted pairs as they are
// (off = 64 or 8 per pair), and once per triplet the activation sums
// sum x and sum x off; the group then adds s (sum x (off + q) - sum x off -
// z sum x).
template <int NJ>
__global__ void __launch_bounds__(kDotThreads) prepass_dotq_kernel(PrepassArgs a) {
  __shared__ float part[NJ * (kDotThreads / 64)];
  const CodeConsts kc = make_code_consts();
  DotBlock b;
  if (!dot_block<NJ>(a, b)) return;
  constexpr int B = 2;
  const int T32 = a.K / 32;
  float acc[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) acc[jj] = 0.f;
  if (b.r < b.rows) {
    const int i = b.base + b.m0 + b.r;
    const int xr = a.gather_div > 0 ? a.sorted_pairs[i] / a.gather_div : i;
    const uint16_t* xp = a.x + (size_t)xr * a.K;
    const uint32_t* qp = a.Vq[b.f] + b.e * a.vq_per_expert + (size_t)b.j0 * T32 * 3;
    const uint32_t* sp = a.Vsz[b.f] + b.e * a.vsz_per_expert + (size_t)b.j0 * (a.K / kGroup);
    const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
    for (int t0 = b.g; t0 < T32; t0 += B * b.G) {
      uint32_t q[B][NJ][3];
      uint2 zw[B][NJ];
      f16x8 xv[B][4];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int tau = t0 + b.G * u;
        const bool in = tau < T32;
        const int tc = in ? tau : 0;
        const uint16_t* xc = xp + 128 * (tc >> 2) + 8 * (tc & 3);
#pragma unroll
        for (int s = 0; s < 4; ++s) xv[u][s] = in ? *(const f16x8*)(xc + 32 * s) : f16x8{};
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          const bool ld = b.j0 + jj < b.rk;       // block-uniform
          const uint32_t* tp = qp + ((size_t)jj * T32 + tc) * 3;
          q[u][jj][0] = ld ? tp[0] : 0u;
          q[u][jj][1] = ld ? tp[1] : 0u;
          q[u][jj][2] = ld ? tp[2] : 0u;
          zw[u][jj] = ld ? *(const uint2*)(sp + (size_t)jj * (a.K / kGroup) + 2 * (tc >> 2)) : uint2{0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        // activation sums of the two groups: sum x and sum x off
        float dx[2], dxo[2];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          float d64 = 0.f, d8 = 0.f;
#pragma unroll
          for (int ss = 0; ss < 2; ++ss)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int s = 2 * gg + ss, pi = 4 * s + v;
              const f16x2 x2 = {xv[u][s][2 * v], xv[u][s][2 * v + 1]};
              if (pair_offset(pi) == 64) d64 = __builtin_amdgcn_fdot2(x2, one2, d64, false);
              else d8 = __builtin_amdgcn_fdot2(x2, one2, d8, false);
            }
          dx[gg] = d64 + d8;
          dxo[gg] = __builtin_fmaf(64.f, d64, 8.f * d8);
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          uint32_t h[16];
          extract_triplet(q[u][jj][0], q[u][jj][1], q[u][jj][2], h, kc);
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            float dq = 0.f;
#pragma unroll
            for (int ss = 0; ss < 2; ++ss)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int s = 2 * gg + ss, pi = 4 * s + v;
                const f16x2 x2 = {xv[u][s][2 * v], xv[u][s][2 * v + 1]};
                dq = __builtin_amdgcn_fdot2(x2, __builtin_bit_cast(f16x2, h[pi]), dq, false);
              }
            const uint32_t w = gg ? zw[u][jj].y : zw[u][jj].x;
            const float sc = half_bits_to_float(w & 0xFFFFu), zp = half_bits_to_float(w >> 16);
            acc[jj] = __builtin_fmaf(sc, __builtin_fmaf(-zp, dx[gg], dq - dxo[gg]), acc[jj]);
          }
        }
      }
    }
  }
  dot_reduce_store<NJ>(acc, b.G, b.rows, b.tout, b.RW, part);
}

template <int NRT, int NWAVES, int UNR, int MT>
__global__ void __launch_bounds__(64 * NWAVES) prepass_kernel(PrepassArgs a) {
  __shared__ float red[NWAVES][MT][NRT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  RowTile rt;
  if (!find_row_tile(a.offsets, a.num_experts, 0, 16 * MT, blockIdx.x, a.rp ? a.rank[0] : nullptr,
                     a.rp ? a.rank[1] : nullptr, &rt))
    return;
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  if ((int)blockIdx.y == a.aux_y) {
    for (int g = m0; g < M && g < m0 + 16 * MT; g += 16) prepass_aux(a, base, g, M, blockIdx.z, gridDim.z);
    return;
  }
  const int RW = a.n_w * a.rp;
  const int tiles_per_w = a.rp / 16;
  const int tr0 = blockIdx.y * NRT;            // first rank tile of this block
  // K chunk of this block: 32-wide steps [s_lo, s_hi)
  const int ksteps = a.K / 32;
  const int s_lo = blockIdx.z * a.ks_steps;
  const int s_hi = s_lo + a.ks_steps < ksteps ? s_lo + a.ks_steps : ksteps;

  // A operand rows of this lane, one per 16-row m-tile
  const uint16_t* xp[MT];
  bool row_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + 16 * mt + (lane & 15);
    row_ok[mt] = m < M;
    int xr = 0;
    if (row_ok[mt]) xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
    xp[mt] = a.x + (size_t)xr * a.K + 8 * (lane >> 4);
  }

  // B operand rows (compensator ranks) of this lane, per rank tile
  const uint16_t* vp[NRT];
  bool vok[NRT];
  bool any = false;
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const int tr = tr0 + t;
    const int f = tr / tiles_per_w;
    const int j = (tr % tiles_per_w) * 16 + (lane & 15);
    vok[t] = j < rt.rank(f);
    any |= (tr % tiles_per_w) * 16 < rt.rank(f);
    vp[t] = a.V[f] + ((size_t)e * a.max_rank + (vok[t] ? j : 0)) * a.K + 8 * (lane >> 4);
  }

  f32x4 acc[MT][NRT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NRT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K steps s = s_lo + wave + NWAVES i, in batches of UNR steps whose loads
  // are all issued before the first product (steps past the chunk are skipped)
  if (any) {
    for (int s0 = s_lo + wave; s0 < s_hi; s0 += UNR * NWAVES) {
      f16x8 xa[UNR][MT], vb[UNR][NRT];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int s = s0 + NWAVES * u;
        const bool in = s < s_hi;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          xa[u][mt] = (in && row_ok[mt]) ? *(const f16x8*)(xp[mt] + 32 * s) : f16x8{};
#pragma unroll
        for (int t = 0; t < NRT; ++t)
          vb[u][t] = (in && vok[t]) ? *(const f16x8*)(vp[t] + 32 * s) : f16x8{};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < NRT; ++t) acc[mt][t] = mfma16x16x32(xa[u][mt], vb[u][t], acc[mt][t]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][mt][t][lane][r] = acc[mt][t][r];
  __syncthreads();

  for (int o = threadIdx.x; o < MT * NRT * 256; o += 64 * NWAVES) {
    const int mt = o / (NRT * 256), t = (o >> 8) % NRT, ln = (o >> 2) & 63, r = o & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) v += red[w][mt][t][ln][r];
    const int row = 16 * mt + 4 * (ln >> 4) + r;  // within the tile
    const int col = (tr0 + t) * 16 + (ln & 15);   // 0..RW-1
    if (m0 + row >= M) continue;
    const size_t o_t = (size_t)(base + m0 + row) * RW + col;
    if (a.tpart) a.tpart[(size_t)blockIdx.z * a.num_pairs * RW + o_t] = v;
    else a.T[o_t] = float_to_half_bits(v);
  }
}

// fp16 V, experts with many rows: block = 128 rows of one expert x every rank
// tile (both families).  The activation tile (128 rows x 128 K per K block)
// goes global -> LDS with global_load_lds_dwordx4 (16-byte chunks
// XOR-swizzled per row, double buffered) and is shared by the four waves;
// wave w owns rank tiles w + 4 u (u < RT) and reads their V fragments straight
// from global memory, one K block ahead.  So the activation rows are read once
// per 128 pairs for all ranks, and each V row once per 128 pairs; no wave
// partials to add (each output has one owner).  grid.z splits K as in
// prepass_kernel (fp32 partials, then the reduce pass).
constexpr int kPtRows = kPrepassTileRows;
constexpr int kPtXBuf = kPtRows * 128;   // halves per staging buffer
constexpr size_t kPtLds = 2 * kPtXBuf * 2;

template <int RT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prepass_tile_kernel(PrepassArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  RowTile rt;
  if (!find_row_tile(a.offsets, a.num_experts, 0, kPtRows, blockIdx.x, a.rp ? a.rank[0] : nullptr,
                     a.rp ? a.rank[1] : nullptr, &rt))
    return;
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  if ((int)blockIdx.y == a.aux_y) {
    for (int g = m0; g < M && g < m0 + kPtRows; g += 16) prepass_aux(a, base, g, M, blockIdx.z, gridDim.z);
    return;
  }
  const int RW = a.n_w * a.rp;
  const int nrt = RW / 16;
  const int tiles_per_w = a.rp / 16;
  const int KB = a.K / 128;
  const int kb_lo = blockIdx.z * (a.ks_steps / 4);
  const int kb_hi = kb_lo + a.ks_steps / 4 < KB ? kb_lo + a.ks_steps / 4 : KB;

  // activation staging (as in the tile GEMM): load j of a wave fills rows
  // 16 j + 4 wave .. + 3; slot p of row r holds column chunk p ^ (r % 16)
  const int srow = 4 * wave + (lane >> 4);
  int xrow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + srow + 16 * j;
    const int i = base + (m < M ? m : m0);
    xrow[j] = a.gather_div > 0 ? a.sorted_pairs[i] / a.gather_div : i;
  }
  const uint16_t* xcol = a.x + 8 * ((lane & 15) ^ (srow & 15));
  auto stage_x = [&](int kb, int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(xcol + (size_t)xrow[j] * a.K + (size_t)kb * 128),
          (__attribute__((address_space(3))) void*)(lds + buf * kPtXBuf + (16 * j + 4 * wave) * 128), 16, 0, 0);
  };
  int xoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xoff[s] = (lane & 15) * 128 + 8 * ((4 * s + (lane >> 4)) ^ (lane & 15));

  // rank tiles of this wave; V rows at or beyond the expert's rank are zero
  const uint16_t* vp[RT];
  bool vok[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const int t = wave + 4 * u;
    const int f = t < nrt ? t / tiles_per_w : 0;
    const int j = t < nrt ? (t % tiles_per_w) * 16 + (lane & 15) : 0;
    vok[u] = t < nrt && j < rt.rank(f);
    vp[u] = a.V[f] + ((size_t)e * a.max_rank + (vok[u] ? j : 0)) * a.K + 8 * (lane >> 4);
  }
  f16x8 vb[RT][4], vn[RT][4];
  auto load_v = [&](int kb, f16x8 (&v)[RT][4]) {
#pragma unroll
    for (int u = 0; u < RT; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 w = *(const f16x8*)(vp[u] + (size_t)kb * 128 + 32 * s);
        v[u][s] = vok[u] ? w : f16x8{};
      }
  };

  f32x4 acc[8][RT];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int u = 0; u < RT; ++u) acc[mt][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kb0 = kb_lo < KB ? kb_lo : KB - 1;   // (chunks are never empty; loads stay in range regardless)
  stage_x(kb0, 0);
  load_v(kb0, vb);
  __syncthreads();   // waits for the staging loads (vmcnt) first
  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    const int buf = (kb - kb_lo) & 1;
    const int kn = kb + 1 < kb_hi ? kb + 1 : kb;   // the last block re-loads its own data
    stage_x(kn, buf ^ 1);
    load_v(kn, vn);
    const uint16_t* xb = lds + buf * kPtXBuf;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const f16x8 xa = *(const f16x8*)(xb + xoff[s] + mt * 16 * 128);
#pragma unroll
        for (int u = 0; u < RT; ++u) acc[mt][u] = mfma16x16x32(xa, vb[u][s], acc[mt][u]);
      }
#pragma unroll
    for (int u = 0; u < RT; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) vb[u][s] = vn[u][s];
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const int t = wave + 4 * u;
    if (t >= nrt) continue;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * (lane >> 4) + r;
        if (m0 + row >= M) continue;
        const size_t o_t = (size_t)(base + m0 + row) * RW + t * 16 + (lane & 15);
        if (a.tpart) a.tpart[(size_t)blockIdx.z * a.num_pairs * RW + o_t] = acc[mt][u][r];
        else a.T[o_t] = float_to_half_bits(acc[mt][u][r]);
      }
  }
}

// T = sum of the K-chunk partials, added in chunk order (fp32), rounded once
// to fp16.  Four elements per thread; n (= P x RW) is a multiple of 32.
__global__ void __launch_bounds__(256) prepass_reduce_kernel(const float* __restrict__ part, int ks, int n,
                                                             uint16_t* __restrict__ T) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= n) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  // eight chunks' loads in flight, added in chunk order
  for (int k0 = 0; k0 < ks; k0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = k0 + u < ks ? *(const f32x4*)(part + (size_t)(k0 + u) * n + i) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s[0] += v[u][0];
      s[1] += v[u][1];
      s[2] += v[u][2];
      s[3] += v[u][3];
    }
  }
  uint2 h;
  h.x = (uint32_t)float_to_half_bits(s[0]) | ((uint32_t)float_to_half_bits(s[1]) << 16);
  h.y = (uint32_t)float_to_half_bits(s[2]) | ((uint32_t)float_to_half_bits(s[3]) << 16);
  *(uint2*)(T + i) = h;
}

// int3 factors, prefill form: block = one 16-row tile of pairs x NRT rank
// tiles of 16 ranks; its NWAVES waves split the 128-wide K blocks.  Per K
// block a lane loads the triplet (row 16 jt + L mod 16, kq = L div 16) of
// each rank tile -- in the V layout that triplet is exactly its matrix-core
// B operand for the block's four 16x16x32 steps -- and the row's two
// scale/zero words, extracts the codes and dequantizes them to fp16
// ((q - z) s, rounded once).  Rank rows at or beyond the expert's rank are
// not loaded (zero operand), so T is exactly 0 there.  Wave partials are
// added in LDS in wave order.
template <int NRT, int NWAVES, int UNR>
__global__ void __launch_bounds__(64 * NWAVES) prepass_q_kernel(PrepassArgs a) {
  __shared__ float red[NWAVES][NRT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const CodeConsts kc = make_code_consts();
  RowTile rt;
  if (!find_tile16(a, &rt)) return;
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  if (is_aux(a)) {
    prepass_aux(a, base, m0, M, blockIdx.y - a.aux_y, a.aux_parts);
    return;
  }
  const int RW = a.n_w * a.rp;
  const int tiles_per_w = a.rp / 16;
  const int tr0 = blockIdx.y * NRT;
  const int KB = a.K / kTileK;
  const int T32 = a.K / 32;

  const int m = m0 + (lane & 15);
  const bool row_ok = m < M;
  int xr = 0;
  if (row_ok) xr = a.gather_div > 0 ? a.sorted_pairs[base + m] / a.gather_div : base + m;
  const uint16_t* xp = a.x + (size_t)xr * a.K + 8 * (lane >> 4);

  const uint32_t* vq[NRT];
  const uint32_t* vs[NRT];
  bool vok[NRT];
  bool any = false;
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const int tr = tr0 + t;
    const int f = tr / tiles_per_w, jt = tr % tiles_per_w;
    const int rk = rt.rank(f);
    const int j = 16 * jt + (lane & 15);
    vok[t] = j < rk;                        // rank <= max_rank: the row is stored
    any |= 16 * jt < rk;
    const int jc = vok[t] ? j : 0;
    vq[t] = a.Vq[f] + e * a.vq_per_expert + ((size_t)jc * T32 + (lane >> 4)) * 3;
    vs[t] = a.Vsz[f] + e * a.vsz_per_expert + (size_t)jc * (a.K / kGroup);
  }

  f32x4 acc[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (any) {
    for (int kb0 = wave; kb0 < KB; kb0 += UNR * NWAVES) {
      f16x8 xa[UNR][4];
      uint32_t q[UNR][NRT][3], zw[UNR][NRT][2];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int kb = kb0 + NWAVES * u;
        const bool in = kb < KB;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xa[u][s] = (in && row_ok) ? *(const f16x8*)(xp + (size_t)kb * kTileK + 32 * s) : f16x8{};
#pragma unroll
        for (int t = 0; t < NRT; ++t) {
          const bool ld = in && vok[t];
          const uint32_t* qp = vq[t] + (size_t)(ld ? kb : 0) * 12;
          q[u][t][0] = ld ? qp[0] : 0u;
          q[u][t][1] = ld ? qp[1] : 0u;
          q[u][t][2] = ld ? qp[2] : 0u;
          const uint2 z2 = ld ? *(const uint2*)(vs[t] + 2 * (size_t)kb) : uint2{0u, 0u};
          zw[u][t][0] = z2.x;
          zw[u][t][1] = z2.y;
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int t = 0; t < NRT; ++t) {
          uint32_t h[16];
          extract_triplet(q[u][t][0], q[u][t][1], q[u][t][2], h, kc);
          const GroupConst g0 = group_const(zw[u][t][0]), g1 = group_const(zw[u][t][1]);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            f16x8 vb = dequant_step(h, s, s < 2 ? g0 : g1);
            if (!vok[t]) vb = f16x8{};
            acc[t] = mfma16x16x32(xa[u][s], vb, acc[t]);
          }
        }
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
    const int row = 4 * (ln >> 4) + r;
    const int col = (tr0 + t) * 16 + (ln & 15);
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
    const milo_weights& w = d->w[f < d->n_w ? f : 0];
    a.V[f] = w.V;
    a.Vq[f] = w.Vq;
    a.Vsz[f] = w.Vsz;
    a.rank[f] = w.rank;
  }
  const bool lrq = d->w[0].lr_format == MILO_LR_INT3;
  a.vq_per_expert = d->max_rank ? milo_lr_v_words(d->max_rank, d->K) : 0;
  a.vsz_per_expert = d->max_rank ? milo_lr_v_sz_words(d->max_rank, d->K) : 0;
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
  a.aux_parts = 1;
  // rows gathered for the small-M kernel: its own experts, or every expert
  // when it takes them all (no tile launch, chunks)
  a.dec_max_rows = (!p.pre_launch && p.dec_ksplit == 1) ? 0x7FFFFFFF : p.dec_max_rows;
  a.tpart = nullptr;
  a.ks_steps = d->K / 32;
  a.num_pairs = d->num_pairs;
  if (per == 1) {                                   // decode
    // int3 V: two ranks per block, one for long rows (more blocks in flight:
    // C2 gate/up 10.7 -> 8.7 us with two instead of four, down 16.8 -> 12.1 us
    // with one)
    const int nj = lrq ? (d->K > 4096 ? 1 : 2) : 1;
    const int rank_groups = p.rp ? d->n_w * p.rp / nj : 0;
    // the gathered-row copy (up to 16 rows of K) is spread over eight blocks
    // per tile, so it does not outlast the rank blocks
    a.aux_y = aux_blocks ? rank_groups : -1;
    a.aux_parts = need_xg ? 8 : 1;
    dim3 grid(p.lr_tiles, rank_groups + aux_blocks * a.aux_parts);
    if (lrq && nj == 1) hipLaunchKernelGGL(prepass_dotq_kernel<1>, grid, dim3(kDotThreads), 0, st, a);
    else if (lrq && nj == 2) hipLaunchKernelGGL(prepass_dotq_kernel<2>, grid, dim3(kDotThreads), 0, st, a);
    else if (lrq) hipLaunchKernelGGL(prepass_dotq_kernel<4>, grid, dim3(kDotThreads), 0, st, a);
    else if (d->K <= 4096) hipLaunchKernelGGL(prepass_dot_kernel<256>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(prepass_dot_kernel<512>, grid, dim3(512), 0, st, a);
    return hip_status(hipGetLastError(), "prepass_dot_kernel launch");
  }
  if (lrq) {
    dim3 grid(p.lr_tiles, rank_blocks + aux_blocks);
    switch (per) {
      case 2: hipLaunchKernelGGL((prepass_q_kernel<2, 4, 2>), grid, dim3(256), 0, st, a); break;
      case 4: hipLaunchKernelGGL((prepass_q_kernel<4, 4, 2>), grid, dim3(256), 0, st, a); break;
      case 8: hipLaunchKernelGGL((prepass_q_kernel<8, 4, 2>), grid, dim3(256), 0, st, a); break;
      default:
        set_error("internal: unsupported rank-tile count %d", per);
        return MILO_ERR_RANK;
    }
    return hip_status(hipGetLastError(), "prepass_q_kernel launch");
  }
  {
    // experts averaging 128 rows or more (plan lr_mt = 8): 128-row tiles with
    // every rank tile per block; otherwise 16-row tiles x groups of at most
    // four 16-rank tiles.  K is split into p.lr_ks chunks (grid.z) when the
    // rows alone give a sparse grid; the chunks' fp32 partials are then added
    // by a reduce pass.
    if (p.lr_ks > 1) a.tpart = (float*)(ws + p.off_tpart);
    if (p.lr_mt == kPtRows / 16) {
      const int tiles = (d->num_pairs + kPtRows - 1) / kPtRows + d->num_experts;
      a.ks_steps = 4 * ((d->K / 128 + p.lr_ks - 1) / p.lr_ks);
      a.aux_y = aux_blocks ? 1 : -1;
      dim3 grid(tiles, 1 + aux_blocks, p.lr_ks);
      if (nrt > 4) hipLaunchKernelGGL(prepass_tile_kernel<2>, grid, dim3(256), kPtLds, st, a);
      else hipLaunchKernelGGL(prepass_tile_kernel<1>, grid, dim3(256), kPtLds, st, a);
    } else {
      const int tpb = per < 4 ? per : 4;
      const int tiles = (d->num_pairs + 15) / 16 + d->num_experts;
      a.aux_y = aux_blocks ? nrt / tpb : -1;
      a.ks_steps = (d->K / 32 + p.lr_ks - 1) / p.lr_ks;
      dim3 grid(tiles, nrt / tpb + aux_blocks, p.lr_ks);
      if (tpb != 2 && tpb != 4) {
        set_error("internal: unsupported rank-tile count %d", per);
        return MILO_ERR_RANK;
      }
      // unsplit K of 32 steps or more: eight waves with all eight of their
      // steps' loads in flight at once (one batch per wave where K <= 2048)
      const bool wide = p.lr_ks == 1 && d->K / 32 >= 32;
      if (tpb == 2 && wide) hipLaunchKernelGGL((prepass_kernel<2, 8, 8, 1>), grid, dim3(512), 0, st, a);
      else if (tpb == 2) hipLaunchKernelGGL((prepass_kernel<2, 4, 4, 1>), grid, dim3(256), 0, st, a);
      else if (wide) hipLaunchKernelGGL((prepass_kernel<4, 8, 8, 1>), grid, dim3(512), 0, st, a);
      else hipLaunchKernelGGL((prepass_kernel<4, 4, 4, 1>), grid, dim3(256), 0, st, a);
    }
    if (p.lr_ks > 1) {
      const int32_t rc = hip_status(hipGetLastError(), "prepass_kernel launch");
      if (rc != MILO_OK) return rc;
      const int n = d->num_pairs * nrt * 16;
      hipLaunchKernelGGL(prepass_reduce_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, a.tpart, p.lr_ks, n,
                         a.T);
      return hip_status(hipGetLastError(), "prepass_reduce_kernel launch");
    }
  }
  return hip_status(hipGetLastError(), "prepass_kernel launch");
}

}  // namespace milo
