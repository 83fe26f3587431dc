// Shared pieces of the two grouped-GEMM kernels (small-M streaming kernel and
// matrix-core tile kernel).
#pragma once
#include "milo_internal.hpp"

namespace milo {

struct GemmArgs {
  const uint16_t* x;
  const int32_t* sorted_pairs;
  const int32_t* offsets;
  const float* slot_w;
  const uint32_t* packed[2];
  const uint32_t* sz[2];
  const uint16_t* U[2];
  const uint32_t* Uq[2];   // int3 compensator: U layout codes and row scale/zero
  const uint32_t* Usz[2];
  const int32_t* rank[2];
  const uint16_t* T;       // fp16 [P][n_w * rp] low-rank pre-pass output
  void* y;
  float* part;             // split-K partial sums
  const float* pw;         // per pair (sorted order): route weight (small-M path)
  int64_t words_per_expert, sz_per_expert, uq_per_expert;
  int lrq;                 // compensator factors are int3
  int N, K, kblocks, n_tiles, gather_div, num_experts, n_w, rp, max_rank;
  int epilogue, ksplit, dec_max_rows, pre_min_rows;
  int m_lo, m_hi;          // row-count range of the experts a decode launch handles
  int poison_over;         // decode launch: NaN-fill the rows of experts above m_hi
  int dec_chunk;           // decode launch: every expert with rows, in chunks of m_hi rows
  int x_bytes_32;          // x (rows x K fp16) spans under 4 GiB: 32-bit row offsets
};

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

struct GemmPlan;
GemmArgs make_gemm_args(const milo_gemm_desc* d, const GemmPlan& p, char* ws);

// Per-(row, group) dequantization constants: d = h * s + c_off for h = off + q.
struct GroupConst {
  float s, c64, c8;
};

__device__ __forceinline__ GroupConst group_const(uint32_t szword) {
  GroupConst g;
  const float s = half_bits_to_float(szword & 0xFFFFu);
  const float z = half_bits_to_float(szword >> 16);
  g.s = s;
  g.c64 = -(64.f + z) * s;
  g.c8 = -(8.f + z) * s;
  return g;
}

// Dequantize the four pairs of MFMA K-step `step` (pairs 4 step .. 4 step + 3)
// of an extracted triplet into one f16x8 operand.
__device__ __forceinline__ f16x8 dequant_step(const uint32_t h[16], int step, const GroupConst& g) {
  uint32_t o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int pi = 4 * step + v;
    o[v] = dequant_pair(h[pi], g.s, pair_offset(pi) == 64 ? g.c64 : g.c8);
  }
  u32x4 u = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(f16x8, u);
}

// fp16 constant B fragments of the folded dequantization: all ones, and the
// per-slot offset (64 or 8) of the pairs of K step `step`; a product with the
// activation fragment gives the rows' sums of x and of x * off.
__device__ __forceinline__ f16x8 ones_frag() {
  const u32x4 u = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  return __builtin_bit_cast(f16x8, u);
}
__device__ __forceinline__ f16x8 offset_frag(int step) {
  u32x4 u;
#pragma unroll
  for (int v = 0; v < 4; ++v) u[v] = pair_offset(4 * step + v) == 64 ? 0x54005400u : 0x48004800u;
  return __builtin_bit_cast(f16x8, u);
}

__device__ __forceinline__ float silu(float u) { return u / (1.f + expf(-u)); }

// Sum of the K splits of a decode launch in split order, then the epilogue.
// Partial sums are [split][expert][n-tile][family][ROWS x 64].
template <int ROWS, int NW, int EPI>
__global__ void __launch_bounds__(256) gemm_split_reduce(GemmArgs a) {
  const int nt = blockIdx.x, e = blockIdx.y;
  const int base = a.offsets[e];
  const int M = a.offsets[e + 1] - base;
  if (M < a.m_lo || M > a.m_hi) return;
  constexpr int kOut = ROWS * 64;
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
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const int o = threadIdx.x + 256 * c;
    const int row = o >> 6, n = o & 63;
    if (row >= M) continue;
    const int i = base + row;
    const int col = nt * kTileRows + n;
    if (EPI == MILO_EPI_ROUTE_SCALE) {
      const int s = a.sorted_pairs[i];
      ((float*)a.y)[(size_t)s * a.N + col] = res[0][c] * a.pw[i];
    } else {
      float v = res[0][c];
      if (EPI == MILO_EPI_SWIGLU) v = silu(v) * res[NW - 1][c];
      ((uint16_t*)a.y)[(size_t)i * a.N + col] = float_to_half_bits(v);
    }
  }
}

}  // namespace milo
