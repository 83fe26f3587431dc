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
  const int32_t* rank[2];
  const uint16_t* T;       // fp16 [P][n_w * rp] low-rank pre-pass output
  void* y;
  float* part;             // split-K partial sums
  const float* pw;         // per pair (sorted order): route weight (small-M path)
  int64_t words_per_expert, sz_per_expert;
  int N, K, kblocks, n_tiles, gather_div, num_experts, n_w, rp, max_rank;
  int epilogue, ksplit, dec_max_rows, pre_min_rows;
};

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

__device__ __forceinline__ float silu(float u) { return u / (1.f + expf(-u)); }

}  // namespace milo
