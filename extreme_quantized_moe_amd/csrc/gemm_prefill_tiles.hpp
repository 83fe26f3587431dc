// Matrix-core (prefill) path of the routed W3A16 + low-rank grouped GEMM:
// the tile kernels, shared by gemm_prefill.hip (64-row tiles and the
// launcher) and gemm_prefill_128.hip (128-row tiles).
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up).  MiLo Kernel: int3 x fp16 GEMM
// with fused dequantization; asynchronous global loads overlap memory with
// compute.  MiLo Algorithm: W_out = W_quant + U V.
//
// Work: (row tile of BM rows, n-tile group), n-tile groups fastest, so the
// blocks that run together share activation rows (L2 hits) while the weights
// stream.  BM = 128 where experts average 256 rows or more, else 64.  One
// block per work item (grid x = n-tile groups, y = row tiles), except the
// 64-row gate/up form, which runs persistent: two blocks per CU walk the
// items of a per-block table of the experts' row tiles (prefix sums in LDS),
// so no block is empty and the expert scan runs once per block.
// Block = BM rows of one expert (pairs in sorted order) x 4 waves.  Each wave
// owns one 64-wide output tile of one weight family (SWIGLU: waves (W1, W3) x
// two n-tiles; otherwise four n-tiles of the one family), so every packed
// weight tile is read and dequantized by exactly one wave.
// Loads: 128-row tiles move activations (BM rows x 128 K, double buffered,
// 16-byte chunks XOR-swizzled per row against bank conflicts) and weights
// (one slot per wave) from global memory straight into LDS with buffer
// loads, so the loop waits only where it says so; 64-row tiles stage the
// activations through LDS and keep a register ring of 2-4 weight stages.
// The next K blocks load while the current one is computed.
// Dequantization: tiles of up to 32 rows fold it into per-group fp32
// corrections (codes reach the matrix cores as exact fp16 off + q); larger
// tiles form (q - z) s in fp32 and round it once to fp16 (v_fma_mix).
// Products on v_mfma_f32_16x16x32_f16 with fp32 accumulation; each K block
// is one branch-free region the scheduler interleaves, issued at raised wave
// priority.
// Epilogue: low-rank term as two more matrix-core K-steps per 32 ranks, then
// SWIGLU through LDS, or fp16 store, or route-weighted fp32 scatter.
#pragma once
#include <type_traits>

#include "gemm_common.hpp"

namespace milo {

// 128-row tile launch (gemm_prefill_128.hip)
int32_t launch_gemm_prefill_128(const GemmArgs& a, int n_w, dim3 grid, hipStream_t st);

// Word 3 of a raw buffer resource (32-bit data format, no swizzle), as used
// for plain byte-addressed buffer loads on this architecture family.
constexpr int kBufRsrcWord3 = 0x00020000;

constexpr int kMaxTileExperts = 256;
constexpr int kXStride = kTileK;         // LDS row stride in halves (256 B; chunks swizzled)
constexpr int kExStride = 68;            // floats per row of the SwiGLU exchange
// LDS of a BM-row block: two staging buffers, or the SwiGLU exchange
constexpr size_t prefill_lds(int bm) {
  return 2 * bm * kExStride * 4 > 2 * bm * kXStride * 2 ? (size_t)2 * bm * kExStride * 4 : (size_t)2 * bm * kXStride * 2;
}

// Weight dequantization, two forms.  Both start from the extracted pair
// h = (off + q): two exact fp16 values.
//
// Packed (two roundings): q = h - off (exact), then fma(q, s, -z s) in packed
// fp16 with -z s rounded to fp16 once per group -- two packed instructions
// per pair of weights; error per weight at most half an fp16 ulp of z s plus
// half an ulp of the result (about 4.8e-4 relative on one product).
//
// Mixed (one rounding): fp16(h s + c) with the group constant c = -(off + z) s
// in fp32; the fused multiply-add runs in fp32 on the fp16 inputs and rounds
// once (v_fma_mixlo / v_fma_mixhi, one instruction per weight), so the matrix
// cores see (q - z) s rounded once (about 2.1e-4 relative on one product).
// Constants: c64 = -s z - 64 s, c8 = c64 + 56 s (fp32), four instructions per
// group.  Measured slower than the packed form (C3 gate/up +7 %, C4 +21 %).
//
// The kernels use the mixed form (tiles of up to two m-tiles fold the
// dequantization out instead, see tile_products_fold): measured layer error
// at 4096 tokens 9.2e-4 with the packed form (bound 1e-3), 4.7e-4 with the
// mixed one.  The packed form is kept for reference and measurement.
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

__device__ __forceinline__ f16x8 dequant_pairs_pk(const uint32_t h4[4], int step, const GroupConstPk& g) {
  const f16x2 off64 = {(_Float16)64.f, (_Float16)64.f}, off8 = {(_Float16)8.f, (_Float16)8.f};
  u32x4 u;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int pi = 4 * step + v;
    const f16x2 q = __builtin_bit_cast(f16x2, h4[v]) - (pair_offset(pi) == 64 ? off64 : off8);
    u[v] = __builtin_bit_cast(uint32_t, q * g.s + g.nzs);
  }
  return __builtin_bit_cast(f16x8, u);
}

struct GroupConstMix {
  float s, c64, c8;
};

__device__ __forceinline__ GroupConstMix group_const_mix(uint32_t szword) {
  const f16x2 sz = __builtin_bit_cast(f16x2, szword);   // (s, z)
  GroupConstMix g;
  g.s = (float)sz[0];
  g.c64 = __builtin_fmaf(-g.s, (float)sz[1], -64.f * g.s);
  g.c8 = __builtin_fmaf(56.f, g.s, g.c64);
  return g;
}

__device__ __forceinline__ f16x8 dequant_pairs_mix(const uint32_t h4[4], int step, const GroupConstMix& g) {
  u32x4 u;
#pragma unroll
  for (int v = 0; v < 4; ++v) u[v] = dequant_pair(h4[v], g.s, pair_offset(4 * step + v) == 64 ? g.c64 : g.c8);
  return __builtin_bit_cast(f16x8, u);
}

// Products of one K block of a wave: the codes of each of the lane's four
// triplets (q: three planes, one word per row group) are extracted once; K
// step s dequantizes its four B operands (one per 16-wide output group, with
// the scale/zero words z; mixed form if MIX) and multiplies them with the A
// fragments of the NMT m-tiles, read from the LDS staging buffer xb at
// xoff[s].
template <int NMT, bool MIX>
__device__ __forceinline__ void tile_products(const u32x4 (&q)[3], const u32x4 (&z)[2], const uint16_t* xb,
                                              const int (&xoff)[4], f32x4 (&acc)[NMT][4], const CodeConsts& kc) {
  uint32_t h[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i) extract_triplet(q[0][i], q[1][i], q[2][i], h[i], kc);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f16x8 wf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = 2 * i + (s >> 1);
      uint32_t h4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) h4[v] = h[i][4 * s + v];
      const uint32_t zw = idx < 4 ? z[0][idx] : z[1][idx - 4];
      if constexpr (MIX) wf[i] = dequant_pairs_mix(h4, s, group_const_mix(zw));
      else wf[i] = dequant_pairs_pk(h4, s, group_const_pk(zw));
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const f16x8 xa = *(const f16x8*)(xb + xoff[s] + mt * 16 * kXStride);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][i] = mfma16x16x32(xa, wf[i], acc[mt][i]);
    }
  }
}

// Products of one K block with the dequantization folded out (for tiles of
// at most two m-tiles, where it costs fewer vector instructions than
// dequantizing every weight, and rounds no weight): the extracted pairs
// (off + q) are exact fp16 B operands; per 64-wide group g of the block the
// accumulator p starts at -(z sum x) - (sum x off) and two products add
// sum x (off + q), so p = sum x (q - z), and acc += s p in fp32.  The row sums
// of x and of x * off are products of the A fragments with constant
// fragments (ones, offsets).
template <int NMT>
__device__ __forceinline__ void tile_products_fold(const u32x4 (&q)[3], const u32x4 (&z)[2], const uint16_t* xb,
                                                   const int (&xoff)[4], f32x4 (&acc)[NMT][4],
                                                   const CodeConsts& kc) {
  f16x8 xa[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[mt][s] = *(const f16x8*)(xb + xoff[s] + mt * 16 * kXStride);
  const f16x8 one = ones_frag();
  f32x4 xs[NMT][2], xo[NMT][2];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      xs[mt][g] = mfma16x16x32(xa[mt][2 * g], one, zero);
      xs[mt][g] = mfma16x16x32(xa[mt][2 * g + 1], one, xs[mt][g]);
      xo[mt][g] = mfma16x16x32(xa[mt][2 * g], offset_frag(2 * g), zero);
      xo[mt][g] = mfma16x16x32(xa[mt][2 * g + 1], offset_frag(2 * g + 1), xo[mt][g]);
    }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h[16];
    extract_triplet(q[0][i], q[1][i], q[2][i], h, kc);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int idx = 2 * i + g;
      const uint32_t w = idx < 4 ? z[0][idx] : z[1][idx - 4];
      const float sc = half_bits_to_float(w & 0xFFFFu);
      const float zp = half_bits_to_float(w >> 16);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_fmaf(-zp, xs[mt][g][r], -xo[mt][g][r]);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const int step = 2 * g + ss;
          const u32x4 u = {h[4 * step], h[4 * step + 1], h[4 * step + 2], h[4 * step + 3]};
          p = mfma16x16x32(xa[mt][step], __builtin_bit_cast(f16x8, u), p);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][i][r] = __builtin_fmaf(sc, p[r], acc[mt][i][r]);
      }
    }
  }
}

// Source addresses of the activation chunks a lane stages: rows
// srow + 16 j (j < NMT) of the tile, gathered through sorted_pairs (or in
// pair order already: no index load); rows past the expert's count take its
// first row.  All index loads are issued before any is used (no dependent
// round trip per row).
template <int NMT>
__device__ __forceinline__ void stage_rows(const GemmArgs& a, int m0, int M, int base, int srow, int lane,
                                           const uint16_t* (&xsrc)[NMT]) {
  int i[NMT], xr[NMT];
#pragma unroll
  for (int j = 0; j < NMT; ++j) {
    const int m = m0 + srow + 16 * j;
    i[j] = base + (m < M ? m : m0);
    xr[j] = i[j];
  }
  if (a.gather_div > 0) {   // uniform: rows in pair order need no index load
#pragma unroll
    for (int j = 0; j < NMT; ++j) xr[j] = a.sorted_pairs[i[j]];
#pragma unroll
    for (int j = 0; j < NMT; ++j) xr[j] /= a.gather_div;
  }
#pragma unroll
  for (int j = 0; j < NMT; ++j) xsrc[j] = a.x + (size_t)xr[j] * a.K + 8 * ((lane & 15) ^ (srow & 15));
}

// The tile's activation row of each lane (tile row l for lane l < 64; rows
// past the expert's count take its first row), loaded ahead of the tile.
__device__ __forceinline__ int tile_row_of_lane(const GemmArgs& a, const RowTile& rt) {
  const int m = rt.m0 + (int)(threadIdx.x & 63);
  const int i = rt.base + (m < rt.rows ? m : rt.m0);
  return a.gather_div > 0 ? a.sorted_pairs[i] / a.gather_div : i;
}

// stage_rows from rows loaded ahead by tile_row_of_lane.
template <int NMT>
__device__ __forceinline__ void stage_rows_pre(const GemmArgs& a, int lane_row, int srow, int lane,
                                               const uint16_t* (&xsrc)[NMT]) {
#pragma unroll
  for (int j = 0; j < NMT; ++j) {
    const int xr = __shfl(lane_row, srow + 16 * j);
    xsrc[j] = a.x + (size_t)xr * a.K + 8 * ((lane & 15) ^ (srow & 15));
  }
}

// Loads of one K block of a wave: its 64 x 128 code tile (three planes), the
// eight scale/zero words of its lane's rows, and its NMT 16-byte chunks of
// the block's activation rows.  Register stages of a ring: everything is a
// plain global load, so the compiler's load counters wait exactly for the
// stage being consumed while the younger stages stay in flight.
template <int NMT>
struct TileStage {
  u32x4 q[3];
  u32x4 z[2];
  u32x4 x[NMT];
};

// Stages in flight: deeper where a K block carries little matrix-core work
// (few rows), as deep as the registers allow at 128 rows.
template <int NMT>
struct TileDepth {
  static constexpr int D = NMT <= 1 ? 4 : (NMT <= 4 ? 3 : 2);
};

// One 32-rank step of the low-rank term of a wave's output tile: the U
// operand (fp16 fragments, or the lane's int3 triplet and the scale/zero
// words of its four rows) and the T fragments of the m-tiles.
template <bool LRQ, int NMT>
struct LrStep {
  f16x8 u[4];
  uint32_t q[3];
  u32x4 sz;
  f16x8 t[NMT];
};

template <bool LRQ, int NMT>
__device__ __forceinline__ void lr_load(const GemmArgs& a, const RowTile& rt, int f, int nt, int s2,
                                        LrStep<LRQ, NMT>& L) {
  const int lane = threadIdx.x & 63;
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  const int RW = a.n_w * a.rp;
  const int j0 = 32 * s2 + 8 * (lane >> 4);
  if constexpr (LRQ) {
    L.sz = *(const u32x4*)(a.Usz[f] + (size_t)e * a.N + nt * kTileRows + 4 * (lane & 15));
    const uint32_t* up = a.Uq[f] + e * a.uq_per_expert + ((size_t)nt * (a.rp / 32) + s2) * 192 + lane;
    L.q[0] = up[0];
    L.q[1] = up[64];
    L.q[2] = up[128];
  } else {
    const int rk = rt.rank(f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = nt * kTileRows + 16 * i + (lane & 15);
      L.u[i] = j0 < rk ? *(const f16x8*)(a.U[f] + ((size_t)e * a.N + n) * a.max_rank + j0) : f16x8{};
    }
  }
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int m = m0 + mt * 16 + (lane & 15);
    const f16x8 tv = *(const f16x8*)(a.T + (size_t)(base + (m < M ? m : m0)) * RW + f * a.rp + j0);
    L.t[mt] = m < M ? tv : f16x8{};
  }
}

template <bool LRQ, int NMT>
__device__ __forceinline__ void lr_apply(const LrStep<LRQ, NMT>& L, int rk, int s2, const CodeConsts& kc,
                                         f32x4 (&acc)[NMT][4]) {
  const int lane = threadIdx.x & 63;
  const int j0 = 32 * s2 + 8 * (lane >> 4);
  f16x8 ub[4];
  if constexpr (LRQ) {
    uint32_t h[16];
    extract_triplet(L.q[0], L.q[1], L.q[2], h, kc);
#pragma unroll
    for (int i = 0; i < 4; ++i) ub[i] = j0 < rk ? dequant_step(h, i, group_const(L.sz[i])) : f16x8{};
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) ub[i] = L.u[i];
  }
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[mt][i] = mfma16x16x32(L.t[mt], ub[i], acc[mt][i]);
}

// Epilogue values loaded when a tile starts, so that their latency hides
// behind the K loop: with ROUTE_SCALE lane l holds the pair index and the
// route weight of tile rows l and 64 + l; with PRE the first 32-rank step of
// the low-rank term is loaded too.
template <bool LRQ, int NMT, bool PRE>
struct TilePre {
  int sp[2];
  float w[2];
  LrStep<LRQ, NMT> lr;
};

// Pair indexes of the tile's rows (first half of TilePre; the weights need
// them, so tile_pre_weights issues their loads later, once they have arrived).
template <int NW, bool LRQ, int NMT, bool PRE>
__device__ __forceinline__ void tile_pre_pairs(const GemmArgs& a, const RowTile& rt, int f, int nt, bool wave_on,
                                               TilePre<LRQ, NMT, PRE>& P) {
  const int lane = threadIdx.x & 63;
  if (NW == 1 && a.epilogue == MILO_EPI_ROUTE_SCALE) {
#pragma unroll
    for (int h = 0; h < (NMT > 4 ? 2 : 1); ++h) {
      const int row = rt.m0 + 64 * h + lane;
      P.sp[h] = row < rt.rows ? a.sorted_pairs[rt.base + row] : 0;
    }
  }
  if constexpr (PRE) {
    if (wave_on && a.rp > 0) lr_load<LRQ, NMT>(a, rt, f, nt, 0, P.lr);
  }
}

template <int NW, bool LRQ, int NMT, bool PRE>
__device__ __forceinline__ void tile_pre_weights(const GemmArgs& a, TilePre<LRQ, NMT, PRE>& P) {
  if (NW == 1 && a.epilogue == MILO_EPI_ROUTE_SCALE) {
#pragma unroll
    for (int h = 0; h < (NMT > 4 ? 2 : 1); ++h) P.w[h] = a.slot_w[P.sp[h]];
  }
}

// After the K loop: the low-rank term and the epilogue of a wave's output
// tile (NMT m-tiles x 64 columns of family f, n-tile nt).
template <int NW, bool LRQ, int NMT, bool PRE>
__device__ __forceinline__ void tile_finish(const GemmArgs& a, const RowTile& rt, uint16_t* lds,
                                            const CodeConsts& kc, f32x4 (&acc)[NMT][4], int f, int nt,
                                            bool wave_on, const TilePre<LRQ, NMT, PRE>& P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = rt.m0, M = rt.rows, base = rt.base;
  // ---- low-rank term: (x V^T) U^T as extra K steps (int3 U: the lane's
  // triplet of each 32-rank U tile is its B operand for the four row groups)
  if (wave_on && a.rp > 0) {
    const int rk = rt.rank(f);
    for (int s2 = 0; s2 < a.rp / 32; ++s2) {
      if (PRE && s2 == 0) {
        lr_apply<LRQ, NMT>(P.lr, rk, 0, kc, acc);
      } else {
        LrStep<LRQ, NMT> L;
        lr_load<LRQ, NMT>(a, rt, f, nt, s2, L);
        lr_apply<LRQ, NMT>(L, rk, s2, kc, acc);
      }
    }
  }

  // ---- epilogue
  if (NW == 2) {
    // waves with f == 1 (W3) hand their tile to the partner wave (wave - 1)
    // rows padded to kExStride floats: the four row groups of a wave's
    // accumulators then fall on different LDS banks
    float* ex = (float*)lds + (wave >> 1) * (NMT * 16 * kExStride);
    if (wave_on && f == 1) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ex[(mt * 16 + 4 * (lane >> 4) + r) * kExStride + 16 * i + (lane & 15)] = acc[mt][i][r];
    }
    __syncthreads();
    if (!wave_on || f == 1) return;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
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
  const bool route = a.epilogue == MILO_EPI_ROUTE_SCALE;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = mt * 16 + 4 * (lane >> 4) + r;
      // row mm's pair and weight from the lane that loaded them (half mt / 4
      // of the tile, lane mm mod 64), read while every lane is active
      int s = 0;
      float w = 0.f;
      if (NW == 1 && route) {
        s = __shfl(P.sp[mt >> 2], mm & 63);
        w = __shfl(P.w[mt >> 2], mm & 63);
      }
      if (m0 + mm >= M) continue;
      const int i_pair = base + m0 + mm;
      if (NW == 1 && route) {
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

// One block's tile: NMT active 16-row m-tiles (the tile's rows, rounded up).
template <int NW, bool LRQ, int NMT, bool X32, int D = TileDepth<NMT>::D, bool ROWPRE = false>
__device__ __forceinline__ void tile_body(const GemmArgs& a, const RowTile& rt, uint16_t* lds,
                                          const CodeConsts& kc, int ng, int lane_row = 0) {
  constexpr int kXBuf = NMT * 16 * kXStride;   // halves per staging buffer
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  const int f = (NW == 2) ? (wave & 1) : 0;
  const int nt = (NW == 2) ? (2 * ng + (wave >> 1)) : (4 * ng + wave);
  const bool wave_on = nt < a.n_tiles;

  // ---- activation staging: lane l of wave w stages, for j < NMT, row
  // 16 j + 4 w + l / 16 of the tile, 16-byte column chunk (l mod 16) XOR
  // (row mod 16), into LDS slot l mod 16 of that row; a fragment read (16
  // rows, one chunk) then hits 16 different slots.  Rows past the expert's
  // count read its first row instead: they only feed outputs that are not
  // stored.
  const int srow = 4 * wave + (lane >> 4);
  const uint16_t* xsrc[NMT];
  if constexpr (ROWPRE) stage_rows_pre<NMT>(a, lane_row, srow, lane, xsrc);
  else stage_rows<NMT>(a, m0, M, base, srow, lane, xsrc);
  const int xdst = srow * kXStride + 8 * (lane & 15);
  // fragment of K step s: row lane % 16 of each m-tile, chunk 4 s + lane / 16
  int xoff[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) xoff[s4] = (lane & 15) * kXStride + 8 * ((4 * s4 + (lane >> 4)) ^ (lane & 15));

  // ---- weights of this wave (a wave without an output tile loads tile 0).
  // Loads are buffer loads: a scalar resource per array, the lane's byte
  // offset in a register, the K block's advance as a scalar offset.
  const int ntc = wave_on ? nt : 0;
  const uint32_t* tbase = a.packed[f] + e * a.words_per_expert + (size_t)ntc * a.kblocks * kTileWords;
  const uint32_t* sbase = a.sz[f] + e * a.sz_per_expert + (size_t)ntc * a.kblocks * kTileSzWords;
  const int KB = a.kblocks;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)tbase, 0, KB * kTileWords * 4, kBufRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)sbase, 0, KB * kTileSzWords * 4, kBufRsrcWord3);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, X32 ? (int)(0xFFFFFFFFu >> 1) : 0, kBufRsrcWord3);
  uint32_t xoff32[NMT];
  if constexpr (X32) {
#pragma unroll
    for (int j = 0; j < NMT; ++j) xoff32[j] = (uint32_t)((const char*)xsrc[j] - (const char*)a.x);
  }
  auto issue = [&](TileStage<NMT>& S, int kb) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
      S.q[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * lane + 1024 * p,
                                                                                kb * kTileWords * 4, 0));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      S.z[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 32 * (lane & 15) + 16 * h,
                                                                                kb * kTileSzWords * 4, 0));
#pragma unroll
    for (int j = 0; j < NMT; ++j) {
      if constexpr (X32)
        S.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff32[j], kb * kTileK * 2, 0));
      else
        S.x[j] = *(const u32x4*)(xsrc[j] + (size_t)kb * kTileK);
    }
  };
  auto put_x = [&](const TileStage<NMT>& S, int buf) {
#pragma unroll
    for (int j = 0; j < NMT; ++j) *(u32x4*)(lds + buf * kXBuf + xdst + 16 * j * kXStride) = S.x[j];
  };

  f32x4 acc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // products of one K block: the codes of each of the lane's four triplets
  // are extracted once; K step s dequantizes its four B operands (one per
  // 16-wide output group) and multiplies them with the m-tiles' A fragments
  auto compute = [&](const TileStage<NMT>& S, int buf) {
    if constexpr (NMT <= 2) tile_products_fold<NMT>(S.q, S.z, lds + buf * kXBuf, xoff, acc, kc);
    else tile_products<NMT, true>(S.q, S.z, lds + buf * kXBuf, xoff, acc, kc);
  };

  // ---- K loop over a ring of D register stages.  Stage j (K block j) sits
  // in slot j mod D: it is issued at the end of block j - D (the slot's
  // previous contents consumed), its activation chunks go to LDS buffer
  // j mod 2 at the end of block j - 1, and block j is computed from them
  // after the barrier.  The loop is unrolled by D so slots are registers.
  // Blocks past the end re-load the last block (never computed): every
  // iteration issues the same loads.
  // epilogue values (pair indexes and weights, the first low-rank step for
  // tiles of up to two m-tiles, where the registers allow) loaded ahead
  constexpr bool kPre = NW == 1 && NMT <= 2;
  TilePre<LRQ, NMT, kPre> pre;
  tile_pre_pairs<NW, LRQ, NMT, kPre>(a, rt, f, nt, wave_on, pre);
  TileStage<NMT> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) issue(ring[d], d < KB ? d : KB - 1);
  put_x(ring[0], 0);
  __syncthreads();
  tile_pre_weights<NW, LRQ, NMT, kPre>(a, pre);
  for (int kb0 = 0; kb0 < KB; kb0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int kb = kb0 + u;
      if (kb < KB) {
        // raised wave priority while a block's products issue, back to
        // normal at the barrier: the two waves sharing a SIMD drift out of
        // phase, one issuing products while the other waits
        __builtin_amdgcn_s_setprio(2);
        if (wave_on) compute(ring[u], kb & 1);
        __builtin_amdgcn_s_setprio(0);
        issue(ring[u], kb + D < KB ? kb + D : KB - 1);
        put_x(ring[(u + 1) % D], (kb + 1) & 1);
        __syncthreads();
      }
    }
  }

  tile_finish<NW, LRQ, NMT, kPre>(a, rt, lds, kc, acc, f, nt, wave_on, pre);
}

// 128-row tiles (eight m-tiles): the accumulators take half the registers,
// so nothing is staged in registers.  Activations and weights both go from
// global memory straight into LDS (global_load_lds: x double buffered, one
// 3.5 KB weight slot per wave: three code planes of 1 KB and the 512-byte
// scale/zero tile), all issued at the start of the previous K block.  Every
// load of the loop is such an LDS transfer, so the compiler inserts no load
// waits of its own; the loop waits explicitly: the wave's own transfers
// (vmcnt 0) before the barrier that ends a block, and its slot read-back
// (lgkmcnt 0) before the slot is refilled.
constexpr int kWSlotHalves = 3584 / 2;    // 3 KB codes + 512 B scale/zero per wave
constexpr size_t prefill_lds_128 = (size_t)2 * 128 * kXStride * 2 + 4 * 3584;

__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

template <int NW, bool LRQ, int NMT, bool X32>
__device__ __forceinline__ void tile_body_lds(const GemmArgs& a, const RowTile& rt, uint16_t* lds,
                                              const CodeConsts& kc, int ng) {
  constexpr int kXBuf = NMT * 16 * kXStride;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = rt.e, m0 = rt.m0, M = rt.rows, base = rt.base;
  const int f = (NW == 2) ? (wave & 1) : 0;
  const int nt = (NW == 2) ? (2 * ng + (wave >> 1)) : (4 * ng + wave);
  const bool wave_on = nt < a.n_tiles;

  // activation staging as in tile_body, but by LDS transfers: load j of a
  // wave fills rows 16 j + 4 wave .. + 3 (lane l: row + l / 16, slot l % 16).
  // Sources as a wave-uniform base plus a per-lane byte offset (32-bit when
  // the activations are under 4 GiB), so that only scalar adds advance them.
  const int srow = 4 * wave + (lane >> 4);
  const uint16_t* xsrc[NMT];
  stage_rows<NMT>(a, m0, M, base, srow, lane, xsrc);
  uint32_t xoff32[NMT];
  if constexpr (X32) {
#pragma unroll
    for (int j = 0; j < NMT; ++j) xoff32[j] = (uint32_t)((const char*)xsrc[j] - (const char*)a.x);
  }
  int xoff[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) xoff[s4] = (lane & 15) * kXStride + 8 * ((4 * s4 + (lane >> 4)) ^ (lane & 15));

  const int ntc = wave_on ? nt : 0;
  const char* tbase = (const char*)(a.packed[f] + e * a.words_per_expert + (size_t)ntc * a.kblocks * kTileWords);
  const char* sbase = (const char*)(a.sz[f] + e * a.sz_per_expert + (size_t)ntc * a.kblocks * kTileSzWords);
  uint16_t* wslot = lds + 2 * kXBuf + wave * kWSlotHalves;
  const int KB = a.kblocks;
  // With activations under 4 GiB every transfer is a buffer load into LDS:
  // a scalar resource per array, the per-lane byte offset in a register and
  // the K block's advance as a scalar offset (no vector address arithmetic).
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, X32 ? (int)(0xFFFFFFFFu >> 1) : 0, kBufRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)tbase, 0, KB * kTileWords * 4, kBufRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)sbase, 0, KB * kTileSzWords * 4, kBufRsrcWord3);
  auto issue = [&](int kb, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int j = 0; j < NMT; ++j) {
      uint16_t* dst = lds + buf * kXBuf + (16 * j + 4 * wave) * kXStride;
      if constexpr (X32) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)dst, 16, xoff32[j],
                                                 kb * kTileK * 2, 0, 0);
      } else {
        dma16((const char*)xsrc[j] + (size_t)kb * kTileK * 2, dst);
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(wslot + 512 * p), 16,
                                               16 * lane + 1024 * p, kb * kTileWords * 4, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(wslot + 1536), 4,
                                             4 * lane, kb * kTileSzWords * 4, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(wslot + 1536 + 128), 4,
                                             4 * lane + 256, kb * kTileSzWords * 4, 0, 0);
  };

  f32x4 acc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one K block: the wave's weights of block kb from its slot into registers
  // (lane l: its 16 bytes of each plane; the scale/zero words of its rows, 32
  // bytes at 32 (l mod 16)), the next block's transfers issued into the slot
  // and the other activation buffer, then the products; the loop is unrolled
  // by two so the buffer offsets are constants
  auto step = [&](int kb, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    u32x4 q[3], z[2];
#pragma unroll
    for (int p = 0; p < 3; ++p) q[p] = *(const u32x4*)(wslot + 512 * p + 8 * lane);
    z[0] = *(const u32x4*)(wslot + 1536 + 16 * (lane & 15));
    z[1] = *(const u32x4*)(wslot + 1536 + 16 * (lane & 15) + 8);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_sched_barrier(0);
    issue(kb + 1 < KB ? kb + 1 : kb, std::integral_constant<int, buf ^ 1>());   // the last block re-loads its own data
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
    if (wave_on) tile_products<NMT, true>(q, z, lds + buf * kXBuf, xoff, acc, kc);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };

  // pair indexes and route weights of the epilogue loaded ahead (the
  // weights once the indexes are in; the first block's wait covers them)
  TilePre<LRQ, NMT, false> pre;
  tile_pre_pairs<NW, LRQ, NMT, false>(a, rt, f, nt, wave_on, pre);
  issue(0, std::integral_constant<int, 0>());
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  tile_pre_weights<NW, LRQ, NMT, false>(a, pre);
  for (int kb = 0; kb < KB; kb += 2) {
    step(kb, std::integral_constant<int, 0>());
    if (kb + 1 < KB) step(kb + 1, std::integral_constant<int, 1>());
  }
  tile_finish<NW, LRQ, NMT, false>(a, rt, lds, kc, acc, f, nt, wave_on, pre);
}

// Row tile `tile` of the 64-row tiling, with the tiles ordered by cost: the
// experts' full tiles first, then their partial last tiles of 33..63, 17..32
// and 1..16 rows, each class in expert order.  The hardware starts blocks in
// index order, so the costliest tiles start first and the cheapest fill the
// tail.  Experts of at most min_rows rows have no tiles.  Block-uniform
// result through LDS; false past the last tile.  The first wave reads the
// offsets and ranks of four experts per lane (up to 256 experts) and scans
// the four classes' tile counts with lane shuffles.  Every thread of the
// block must call it.
__device__ __forceinline__ bool find_row_tile64_by_cost(const GemmArgs& a, int tile, RowTile* out) {
  __shared__ int res[6];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, E = a.num_experts;
    const int32_t* rk0 = a.rp ? a.rank[0] : a.offsets;   // valid dummy when unused
    const int32_t* rk1 = a.rp ? a.rank[1] : a.offsets;
    int o0[4], o1[4], r0[4], r1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * lane + c;
      const int ec = e < E ? e : E - 1;
      o0[c] = a.offsets[ec];
      o1[c] = a.offsets[ec + 1];
      r0[c] = rk0[ec];
      r1[c] = rk1[ec];
    }
    if (lane == 0) res[0] = -1;
    int n[4][4], sum[4] = {0, 0, 0, 0};   // [class][expert of the lane]
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int M = 4 * lane + c < E ? o1[c] - o0[c] : 0;
      const bool in = M > a.pre_min_rows;
      const int rem = M % 64;
      n[0][c] = in ? M / 64 : 0;
      n[1][c] = in && rem > 32 ? 1 : 0;
      n[2][c] = in && rem > 16 && rem <= 32 ? 1 : 0;
      n[3][c] = in && rem > 0 && rem <= 16 ? 1 : 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) sum[k] += n[k][c];
    }
    int before = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int inc = sum[k];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      int first = before + inc - sum[k];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (n[k][c] > 0 && tile >= first && tile < first + n[k][c]) {
          const int M = o1[c] - o0[c];
          res[0] = 4 * lane + c;
          res[1] = k == 0 ? (tile - first) * 64 : (M / 64) * 64;
          res[2] = M;
          res[3] = o0[c];
          res[4] = a.rp ? r0[c] : 0;
          res[5] = a.rp ? r1[c] : 0;
        }
        first += n[k][c];
      }
      before += __shfl(inc, 63);
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

template <int NW, bool LRQ, int BM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_prefill_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const CodeConsts kc = make_code_consts();
  RowTile rt;
  const bool found = BM == 64 ? find_row_tile64_by_cost(a, blockIdx.y, &rt)
                              : find_row_tile(a.offsets, a.num_experts, a.pre_min_rows, BM, blockIdx.y,
                                              a.rp ? a.rank[0] : nullptr, a.rp ? a.rank[1] : nullptr, &rt);
  if (!found) return;
  if constexpr (BM == 64) {
    // only the tile's own rows: fewer products and staged rows for the
    // small experts (a 3-row expert costs one m-tile, not four)
    const int rows = rt.rows - rt.m0;
    if (a.x_bytes_32) {
      if (rows <= 16) tile_body<NW, LRQ, 1, true>(a, rt, lds, kc, blockIdx.x);
      else if (rows <= 32) tile_body<NW, LRQ, 2, true>(a, rt, lds, kc, blockIdx.x);
      else tile_body<NW, LRQ, 4, true>(a, rt, lds, kc, blockIdx.x);
    } else {
      tile_body<NW, LRQ, 4, false>(a, rt, lds, kc, blockIdx.x);
    }
  } else {
    if (a.x_bytes_32) tile_body_lds<NW, LRQ, BM / 16, true>(a, rt, lds, kc, blockIdx.x);
    else tile_body_lds<NW, LRQ, BM / 16, false>(a, rt, lds, kc, blockIdx.x);
  }
}


// 64-row tiles, persistent: a grid of two blocks per compute unit walks the
// work items (row tile, n-tile group), n-tile groups fastest (consecutive
// items share activation rows).  The row tiles are listed once per block, by
// cost: the experts' full 64-row tiles first, then their partial last tiles
// of 33..63, 17..32 and 1..16 rows (four, two and one m-tiles), each class as
// prefix sums over the experts in LDS; an item finds its tile by binary
// search.  Items are dealt in rounds of one per block, every other round in
// reverse block order, so a block that took one of the costliest items of a
// round takes one of the cheapest of the next (a Zipf-skewed routing leaves
// about 1.5 items per block, where a plain round robin gives some blocks two
// costly items and others one cheap one; C4 gate/up 83 -> 78 us).  Dealing
// a round's consecutive items to the blocks of one XCD instead (blocks are
// placed on the eight XCDs round robin) was slower (84 us): it puts a round's
// costliest items on one XCD.  The next item's activation row indexes are
// loaded while the current item runs.  No block starts past the last item,
// and the expert scan runs once per block instead of once per tile.  With
// three tile shapes in one loop the registers allow two stages in flight for
// the 2- and 4-m-tile shapes; that suits the gate/up form (two weight
// families per wave), while
// the one-family form keeps its three stages in the one-tile-per-block
// kernel, measured faster there.
template <int NW, bool LRQ>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_prefill_persistent(GemmArgs a, int n_groups) {
  extern __shared__ __align__(16) uint16_t lds[];
  // tab[0]: full tiles; tab[1..3]: partial last tiles of 33..63, 17..32, 1..16 rows
  __shared__ int tab[4][kMaxTileExperts + 1];
  __shared__ int e_base[kMaxTileExperts], e_rows[kMaxTileExperts], e_rk0[kMaxTileExperts],
      e_rk1[kMaxTileExperts];
  const CodeConsts kc = make_code_consts();
  const int E = a.num_experts;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int32_t* rk0 = a.rp ? a.rank[0] : a.offsets;   // valid dummy when unused
    const int32_t* rk1 = a.rp ? a.rank[1] : a.offsets;
    int o0[4], o1[4], r0[4], r1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * lane + c;
      const int ec = e < E ? e : E - 1;
      o0[c] = a.offsets[ec];
      o1[c] = a.offsets[ec + 1];
      r0[c] = rk0[ec];
      r1[c] = rk1[ec];
    }
    int n[4][4], sum[4] = {0, 0, 0, 0};   // [class][expert of the lane]
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * lane + c;
      const int M = e < E ? o1[c] - o0[c] : 0;
      const bool in = M > a.pre_min_rows;
      const int rem = M % 64;
      n[0][c] = in ? M / 64 : 0;
      n[1][c] = in && rem > 32 ? 1 : 0;
      n[2][c] = in && rem > 16 && rem <= 32 ? 1 : 0;
      n[3][c] = in && rem > 0 && rem <= 16 ? 1 : 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) sum[k] += n[k][c];
      if (e < E) {
        e_base[e] = o0[c];
        e_rows[e] = M;
        e_rk0[e] = a.rp ? r0[c] : 0;
        e_rk1[e] = a.rp ? r1[c] : 0;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int inc = sum[k];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      int r = inc - sum[k];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * lane + c;
        if (e < E) tab[k][e] = r;
        r += n[k][c];
      }
      if (lane == 63) tab[k][E] = inc;   // the totals (E may be 256, past every lane's experts)
    }
  }
  __syncthreads();
  const int T0 = tab[0][E], T1 = T0 + tab[1][E], T2 = T1 + tab[2][E], T3 = T2 + tab[3][E];
  const int n_items = T3 * n_groups;
  // the last expert with tab[e] <= t (experts without tiles of the class
  // share their successor's start and are skipped)
  auto find = [&](const int* t_, int t) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (t_[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  const int G = gridDim.x, b = blockIdx.x;
  auto item = [&](int round) { return round * G + ((round & 1) ? G - 1 - b : b); };
  auto lookup = [&](int w, RowTile& rt) {
    const int tile = w / n_groups;
    if (tile < T0) {
      rt.e = find(tab[0], tile);
      rt.m0 = (tile - tab[0][rt.e]) * 64;
    } else {
      const int k = tile < T1 ? 1 : (tile < T2 ? 2 : 3);
      const int first = k == 1 ? T0 : (k == 2 ? T1 : T2);
      rt.e = find(tab[k], tile - first);
      rt.m0 = (e_rows[rt.e] / 64) * 64;
    }
    rt.rows = e_rows[rt.e];
    rt.base = e_base[rt.e];
    rt.rank0 = e_rk0[rt.e];
    rt.rank1 = e_rk1[rt.e];
  };
  // each item's activation row indexes are loaded while the previous item
  // runs (one register per lane), so an item starts with its first loads
  RowTile nrt;
  int nrow = 0;
  if (item(0) < n_items) {
    lookup(item(0), nrt);
    nrow = tile_row_of_lane(a, nrt);
  }
  for (int round = 0;; ++round) {
    const int w = item(round);
    if (w >= n_items) break;
    const int ng = w % n_groups;
    const RowTile rt = nrt;
    const int row = nrow;
    if (item(round + 1) < n_items) {
      lookup(item(round + 1), nrt);
      nrow = tile_row_of_lane(a, nrt);
    }
    // the launcher takes this kernel only when the activations fit 32-bit
    // offsets
    if (rt.rows - rt.m0 <= 16) tile_body<NW, LRQ, 1, true, TileDepth<1>::D, true>(a, rt, lds, kc, ng, row);
    else if (rt.rows - rt.m0 <= 32) tile_body<NW, LRQ, 2, true, 2, true>(a, rt, lds, kc, ng, row);
    else tile_body<NW, LRQ, 4, true, 2, true>(a, rt, lds, kc, ng, row);
    __syncthreads();   // the next item reuses the LDS
  }
}

}  // namespace milo
