// Internal declarations shared by the libmilo translation units (device
// helpers, kernel launchers).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/milo.h"

namespace milo {

// ---------------------------------------------------------------- types
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTileRows = 64;      // rows (output features) per packed tile
constexpr int kTileK = 128;        // input features per packed tile
constexpr int kTileWords = 768;    // 3 planes x 64 lanes x 4 words
constexpr int kTileSzWords = 128;  // 64 rows x 2 groups
constexpr int kGroup = 64;
constexpr int kMaxRank = 64;
constexpr int kDecodeMaxRows = 32;  // largest expert row count of the small-M path
constexpr int kDecodeChunkRows = 128; // largest row bound of a chunked small-M plan
constexpr int64_t kSmallMatrixElems = (int64_t)1 << 22;  // N x K at most: mid-sized experts take the tile kernel
constexpr int kPrepassTileRows = 128;  // rows per block of the fp16 prefill pre-pass for large experts
constexpr int kPrepassBlocks = 512; // the fp16 prefill pre-pass splits K until its grid has about this many blocks

// Per-pair constant offsets of the "off + q" float16 encoding produced by the
// code extraction (see dequant_triplet): pair pi of a triplet holds codes at
// mantissa bits 4..6 (value 64 + q) or 7..9 (value 8 + q).
__host__ __device__ constexpr int pair_offset(int pi) {
  return (pi == 15) ? 64 : ((pi % 5 == 2 || pi % 5 == 4) ? 8 : 64);
}

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Masks and float16 magic words of the code extraction, held in registers.
// They are produced by inline asm so that the compiler cannot fold them back
// into literals (gfx9 VOP3 encodings take no literal, and two literal
// operands would split every v_and_or_b32 into two instructions).  Only
// these definitions are asm: every extraction op is ordinary code, so the
// compiler's hazard tracking sees the VALU writes that feed the matrix cores
// (a matrix instruction reads its sources a fixed number of wait states after
// a VALU write, and the compiler cannot insert them for results of inline asm).
struct CodeConsts {
  uint32_t lo, hi, b4, b5, b6;   // SGPR masks
  uint32_t m64, m8;              // VGPR magic words: float16 64.0 / 8.0 in both halves
};

__device__ __forceinline__ CodeConsts make_code_consts() {
  CodeConsts k;
  asm volatile("s_mov_b32 %0, 0x00700070" : "=s"(k.lo));   // bits 4..6 of each half
  asm volatile("s_mov_b32 %0, 0x03800380" : "=s"(k.hi));   // bits 7..9 of each half
  asm volatile("s_mov_b32 %0, 0x00100010" : "=s"(k.b4));
  asm volatile("s_mov_b32 %0, 0x00200020" : "=s"(k.b5));
  asm volatile("s_mov_b32 %0, 0x00400040" : "=s"(k.b6));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(k.m64));
  asm volatile("v_mov_b32 %0, 0x48004800" : "=v"(k.m8));
  return k;
}

// (a & mask) | b: one v_and_or_b32 with mask in an SGPR and b in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b) {
  return (a & mask) | b;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
}

// Extract the 16 code pairs of one layout-v1 triplet (words w0, w1, w2) into
// float16x2 words holding (off + q_even, off + q_odd) with off = pair_offset.
__device__ __forceinline__ void extract_triplet(uint32_t w0, uint32_t w1, uint32_t w2,
                                                uint32_t out[16], const CodeConsts& k) {
  uint32_t w[3] = {w0, w1, w2};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    uint32_t a = w[p];
    uint32_t sh = a >> 6;
    out[5 * p + 0] = and_or(a << 3, k.lo, k.m64);   // bits 1..3  -> 4..6
    out[5 * p + 1] = and_or(a, k.lo, k.m64);        // bits 4..6
    out[5 * p + 2] = and_or(a, k.hi, k.m8);         // bits 7..9
    out[5 * p + 3] = and_or(sh, k.lo, k.m64);       // bits 10..12 -> 4..6
    out[5 * p + 4] = and_or(sh, k.hi, k.m8);        // bits 13..15 -> 7..9
  }
  uint32_t s = and_or(w0 << 4, k.b4, k.m64);
  s = and_or(w1 << 5, k.b5, s);
  out[15] = and_or(w2 << 6, k.b6, s);
}

// The four code pairs of MFMA K-step `step` (pairs 4 step .. 4 step + 3) of
// one layout-v1 triplet, extracted on their own (the same values as
// extract_triplet's out[4 step .. 4 step + 3]); for callers that cannot keep
// all sixteen extracted pairs of a triplet live at once.
__device__ __forceinline__ void extract_step(uint32_t w0, uint32_t w1, uint32_t w2, int step, uint32_t out[4],
                                             const CodeConsts& k) {
  const uint32_t w[3] = {w0, w1, w2};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int pi = 4 * step + v;
    if (pi == 15) {
      uint32_t s = and_or(w0 << 4, k.b4, k.m64);
      s = and_or(w1 << 5, k.b5, s);
      out[v] = and_or(w2 << 6, k.b6, s);
      continue;
    }
    const uint32_t a = w[pi / 5];
    switch (pi % 5) {
      case 0: out[v] = and_or(a << 3, k.lo, k.m64); break;
      case 1: out[v] = and_or(a, k.lo, k.m64); break;
      case 2: out[v] = and_or(a, k.hi, k.m8); break;
      case 3: out[v] = and_or(a >> 6, k.lo, k.m64); break;
      default: out[v] = and_or(a >> 6, k.hi, k.m8); break;
    }
  }
}

// (off + q) -> (q - z) * s as float16, computed as fma(h, s, -(off + z) s) in
// float32 and rounded once.
__device__ __forceinline__ uint32_t dequant_pair(uint32_t h, float s, float c) {
  f16x2 v = __builtin_bit_cast(f16x2, h);
  f16x2 r;
  r[0] = (_Float16)__builtin_fmaf((float)v[0], s, c);
  r[1] = (_Float16)__builtin_fmaf((float)v[1], s, c);
  return __builtin_bit_cast(uint32_t, r);
}

// Row tile `tile` when the experts with more than `min_rows` rows are cut
// into tiles of `rows_per_tile` rows, expert by expert: its expert, first row
// within the expert, the expert's row count and first pair, and the expert's
// compensator rank in the two weight families (0 where the rank array is
// null).  Block-uniform result; returns false past the last tile.  The first
// wave issues every load at once (offsets and ranks of up to 256 experts;
// indexes are clamped instead of predicated, since a predicated load per
// expert group is compiled to its own branch with a wait after it), scans
// the per-expert tile counts with lane shuffles, and the lane holding the
// tile publishes it through LDS, so callers need no further dependent load
// for these values.  Every thread of the block must call it.
struct RowTile {
  int e, m0, rows, base, rank0, rank1;
  // by selection, not indexing: a runtime index would put the struct in memory
  __device__ __forceinline__ int rank(int f) const { return f ? rank1 : rank0; }
};

__device__ __forceinline__ bool find_row_tile(const int32_t* __restrict__ offsets, int num_experts,
                                              int min_rows, int rows_per_tile, int tile,
                                              const int32_t* __restrict__ rank0,
                                              const int32_t* __restrict__ rank1, RowTile* out) {
  __shared__ int res[6];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int32_t* rk0 = rank0 ? rank0 : offsets;   // valid dummy, values unused
    const int32_t* rk1 = rank1 ? rank1 : offsets;
    int o0[4], m[4], r0[4], r1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {          // up to 256 experts
      const int e = 64 * c + lane;
      const int ec = e < num_experts ? e : num_experts - 1;
      o0[c] = offsets[ec];
      m[c] = offsets[ec + 1];
      r0[c] = rk0[ec];
      r1[c] = rk1[ec];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool in = 64 * c + lane < num_experts;
      m[c] = in ? m[c] : o0[c];            // no rows past the last expert
      r0[c] = rank0 ? r0[c] : 0;
      r1[c] = rank1 ? r1[c] : 0;
    }
    if (lane == 0) res[0] = -1;
    int before = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (64 * c >= num_experts) break;
      m[c] -= o0[c];
      const int nt = m[c] > min_rows ? (m[c] + rows_per_tile - 1) / rows_per_tile : 0;
      int incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      const int first = before + incl - nt;
      if (nt > 0 && tile >= first && tile < first + nt) {
        res[0] = 64 * c + lane;
        res[1] = (tile - first) * rows_per_tile;
        res[2] = m[c];
        res[3] = o0[c];
        res[4] = r0[c];
        res[5] = r1[c];
      }
      before += __shfl(incl, 63);
    }
  }
  __syncthreads();
  out->e = res[0];
  out->m0 = res[1];
  out->rows = res[2];
  out->base = res[3];
  out->rank0 = res[4];
  out->rank1 = res[5];
  return out->e >= 0;
}

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
int32_t hip_status(hipError_t e, const char* what);

// launchers (return MILO_OK or MILO_ERR_HIP)
int32_t launch_quantize(const float* W, int64_t rows, int64_t K, int group, uint8_t* codes,
                        uint16_t* scale, uint16_t* zero, hipStream_t st);
int32_t launch_pack_lr(const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                       const uint8_t* u_codes, const uint16_t* u_scale, const uint16_t* u_zero,
                       int64_t N, int64_t K, int rank, int max_rank, uint32_t* vq, uint32_t* vsz,
                       uint32_t* uq, uint32_t* usz, hipStream_t st);
int32_t launch_hqq(const float* W, int64_t rows, int64_t K, int iters, double p, double beta, double kappa,
                   uint8_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t st);
int32_t launch_pack(const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                    int64_t rows, int64_t K, uint32_t* packed, uint32_t* sz, hipStream_t st);
int32_t launch_route(const float* logits, int T, int E, int k, int S, int renorm,
                     int32_t* ids, float* w, float* slot_w, int32_t* sorted_pairs,
                     int32_t* pair_pos, int32_t* offsets, void* ws, hipStream_t st);
int32_t launch_combine(const float* y, int T, int slots, int H, uint16_t* out, hipStream_t st);

// compensator construction (builder.hip)
size_t svd_workspace_bytes(int64_t N, int64_t K, int l);
size_t build_workspace_bytes(int64_t N, int64_t K, int l);
int32_t run_lowrank_svd(const float* R, int64_t N, int64_t K, int r, int l, int q, const float* omega_t,
                        float* U, float* V, float* sigma, char* ws, hipStream_t st);
int32_t run_build(const float* W, int64_t N, int64_t K, int r, int iters, int l, int q, const float* omega,
                  int quantizer, uint8_t* codes, uint16_t* scale, uint16_t* zero, float* U, float* V,
                  float* sigma, char* ws, hipStream_t st);

// adaptive rank policy (rank_policy.hip)
size_t kurtosis_workspace_bytes(int64_t count);
int32_t launch_kurtosis(const float* W, int64_t count, int64_t elems, double* kurt, double* mean_out,
                        char* ws, hipStream_t st);
int32_t launch_expert_counts(const int32_t* offsets, int E, int64_t* counts, hipStream_t st);
void rank_policy_host(const double* kurt, const double* freq, const int32_t* dense, int n, int total_rank,
                      int r_min, int r_max, int step, int32_t* ranks);

// Resolved plan of one grouped-GEMM call (host side).
struct GemmPlan {
  int n_tiles;       // N / 64
  int kblocks;       // K / 128
  int rp;            // compensator rank padded to 32 (0 = no compensator)
  int lr_tiles_per_block;  // rank tiles (16 ranks) per pre-pass block
  int lr_tiles;      // grid.x of the low-rank pre-pass (16-row tiles)
  int lr_mt;         // fp16 prefill-form pre-pass: 16-row m-tiles per block (8: the 128-row tile kernel)
  int lr_ks;         // fp16 prefill-form pre-pass: K chunks (fp32 partials + reduce when > 1)
  int dec_mt;        // 16-row m-tiles of the small-M kernel (0 = not launched)
  int dec_max_rows;  // experts with at most this many rows use the small-M kernel
  int dec_ksplit;    // split-K factor of the small-M kernel
  int dec_blocks;    // persistent grid of the small-M kernel
  int pre_launch;    // launch the tile kernel
  int pre_tiles;     // grid.y bound of the tile kernel (row tiles)
  int pre_bm;        // rows per block of the tile kernel (64 or 128)
  int pre_slots;     // persistent grid of the 64-row tile kernel (two blocks per compute unit)
  int dec_chunked;   // planned as small-M only with experts above 32 rows in chunks
  // workspace carve-up (byte offsets)
  size_t off_t, off_xg, off_pw, off_dec_part, off_tpart, total;
};
int32_t plan_gemm(const milo_gemm_desc* d, GemmPlan* p);
int32_t launch_lowrank(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st);
int32_t launch_gemm_decode(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st);
int32_t launch_gemm_prefill(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st);

}  // namespace milo
