// Softmax top-k routing and the stable expert sort of (token, slot) pairs.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), Background: an MoE layer activates
// only a subset of its experts per token.  The router itself is not given on
// the pages; this is the usual softmax top-k (ties -> lower expert id).
//
// Three phases, each deterministic:
//   1. route_topk  (one thread per token up to 16 experts, four above;
//      256 tokens per block): top-k,
//      weights, and per-block stable ranks of each slot among the slots of the
//      same expert, from an LDS bitmap [expert][token-in-block].
//   2. route_scan  (one block): per expert, exclusive prefix of the block
//      counts; exclusive prefix over experts -> offsets.
//   3. route_scatter: final positions.
// With a single token block, phase 1 does all three (one launch), except for
// rows wider than 16 experts: then route_topk_wave selects on one wave per
// token across many compute units and route_sort_block ranks, scans and
// scatters in one block (two launches).
#include "milo_internal.hpp"

namespace milo {

constexpr int kRouteBlock = 256;                 // tokens per block
constexpr int kMaxExperts = 256;
constexpr int kBitWords = kRouteBlock / 32;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = 16;

__device__ __forceinline__ int slot_expert(const int32_t* ids_row, int j, int k, int E) {
  return j < k ? ids_row[j] : E + (j - k);
}

// Top-k of one token's logits by one thread (up to 16 experts): k passes,
// pass j picks the largest logit (lowest id on ties) among the experts not
// picked before; also the row maximum and the softmax denominator.  The row
// is held in registers (NE >= E; all loads issued at once).
template <int NE, int MK>
__device__ __forceinline__ void topk_regs(const float* row, int E, int k, float (&bv)[MK],
                                          int (&bi)[MK], float& mx, float& den) {
  float v[NE];
  if (E == NE && ((uintptr_t)row & 15) == 0) {
    // whole 16-byte vectors: a quarter of the cache-line requests of scalar
    // loads (the rows of neighbouring threads are E floats apart)
#pragma unroll
    for (int e = 0; e < NE; e += 4) {
      const float4 q = *(const float4*)(row + e);
      v[e] = q.x, v[e + 1] = q.y, v[e + 2] = q.z, v[e + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < NE; ++e) v[e] = e < E ? row[e] : -INFINITY;
  }
  mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < NE; ++e)
    if (e < E) mx = fmaxf(mx, v[e]);
  uint64_t taken = 0;
#pragma unroll
  for (int j = 0; j < MK; ++j) {
    bv[j] = -INFINITY;
    bi[j] = -1;
    if (j < k) {
      float best = -INFINITY;
      int bidx = -1;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const bool ok = e < E && !((taken >> e) & 1ull);
        if (ok && (bidx < 0 || v[e] > best)) {
          best = v[e];
          bidx = e;
        }
      }
      bv[j] = best;
      bi[j] = bidx;
      taken |= 1ull << bidx;
    }
  }
  den = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e)
    if (e < E) den += expf(v[e] - mx);
}

// Top-k of one token's logits by its LANES threads (1 or 4).  Thread q of
// the token holds experts [q NL, (q + 1) NL) in registers (16-byte loads when
// the row is whole vectors: the threads read the row contiguously), takes its
// own top-k (k passes, strictly greater replaces, so ties keep the lower id),
// and with four threads the sorted lists are merged k times by a max over the
// four (larger value, then lower id), the winner dropping its head.  The
// softmax denominator: each thread's sum of exp(v - max) over its experts,
// then (with four) the partial sums as (t0 + t1) + (t2 + t3).
template <int LANES, int NL, int MK>
__device__ __forceinline__ void topk_lanes(const float* row, int E, int k, int q, float (&bv)[MK],
                                           int (&bi)[MK], float& den) {
  float v[NL];
  const int e0 = q * NL;
  if (E == LANES * NL && NL % 4 == 0 && ((uintptr_t)row & 15) == 0) {
#pragma unroll
    for (int e = 0; e < NL; e += 4) {
      const float4 x = *(const float4*)(row + e0 + e);
      v[e] = x.x, v[e + 1] = x.y, v[e + 2] = x.z, v[e + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < NL; ++e) v[e] = e0 + e < E ? row[e0 + e] : -INFINITY;
  }
  // own list, best first; entries past the own experts are (-inf, E + 1)
  float lv[MK];
  int li[MK];
  uint64_t taken = 0;
#pragma unroll
  for (int j = 0; j < MK; ++j) {
    lv[j] = -INFINITY;
    li[j] = E + 1;
    if (j < k) {
      int bidx = -1;
      float best = -INFINITY;
#pragma unroll
      for (int e = 0; e < NL; ++e) {
        const bool ok = e0 + e < E && !((taken >> e) & 1ull);
        if (ok && (bidx < 0 || v[e] > best)) {
          best = v[e];
          bidx = e;
        }
      }
      if (bidx >= 0) {
        lv[j] = best;
        li[j] = e0 + bidx;
        taken |= 1ull << bidx;
      }
    }
  }
  if constexpr (LANES == 1) {
#pragma unroll
    for (int j = 0; j < MK; ++j) {
      bv[j] = j < k ? lv[j] : -INFINITY;
      bi[j] = j < k ? li[j] : -1;
    }
  }
  // merge the four lists
#pragma unroll
  for (int j = 0; j < MK; ++j) {
    if (LANES == 1) break;
    bv[j] = -INFINITY;
    bi[j] = -1;
    if (j < k) {
      float cv = lv[0];
      int ci = li[0];
#pragma unroll
      for (int o = 1; o <= 2; o <<= 1) {
        const float ov = __shfl_xor(cv, o);
        const int oi = __shfl_xor(ci, o);
        if (ov > cv || (ov == cv && oi < ci)) {
          cv = ov;
          ci = oi;
        }
      }
      bv[j] = cv;
      bi[j] = ci;
      const bool mine = li[0] == ci;
#pragma unroll
      for (int u = 0; u + 1 < MK; ++u) {
        lv[u] = mine ? lv[u + 1] : lv[u];
        li[u] = mine ? li[u + 1] : li[u];
      }
      if (mine) {
        lv[MK - 1] = -INFINITY;
        li[MK - 1] = E + 1;
      }
    }
  }
  const float mx = bv[0];
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < NL; ++e)
    if (e0 + e < E) part += expf(v[e] - mx);
  if (LANES == 4) {
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
  }
  den = part;
}

// Block-wide exclusive scan of one int per thread (blockDim == 256).
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < kRouteBlock; off <<= 1) {
    int add = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += add;
    __syncthreads();
  }
  const int incl = lds[tid];
  *total = lds[kRouteBlock - 1];
  __syncthreads();
  return incl - v;
}

// NV: experts per token row this instantiation handles (LANES = 1: 8 or 16
// in registers; LANES = 4: 32, 64, 128 or 256, a quarter per thread); MK and
// MS bound k and the slots per token (k + shared).  One width and bound per
// kernel keeps each kernel's code small: a single block runs it cold from the
// instruction cache, and the fully unrolled slot loops are most of the code
// (top-2 over 8 experts: 2655 instructions with bounds 8 / 16).
template <int LANES, int NV, int MK, int MS>
__global__ void __launch_bounds__(LANES * kRouteBlock)
route_topk(const float* __restrict__ logits, int T, int E, int k, int S, int renorm,
           int32_t* __restrict__ ids, float* __restrict__ topw, float* __restrict__ slot_w,
           int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
           int32_t* __restrict__ offsets, int32_t* __restrict__ block_counts) {
  __shared__ uint32_t bits[kMaxExperts][kBitWords];
  __shared__ int scan_lds[kRouteBlock];
  const int tid = threadIdx.x;
  const int tl = tid / LANES, q = tid % LANES;    // token in block, its thread
  const int t = blockIdx.x * kRouteBlock + tl;
  const int ET = E + S, slots = k + S;
  for (int x = tid; x < ET * kBitWords; x += LANES * kRouteBlock) (&bits[0][0])[x] = 0u;
  __syncthreads();

  // per-thread arrays are indexed only by unrolled loop counters (registers);
  // slot j of a token is handled by its thread j % LANES
  int my_ids[MS];
  int rank[MS];
#pragma unroll
  for (int j = 0; j < MS; ++j) {
    my_ids[j] = 0;
    rank[j] = 0;
  }
  const bool live = t < T;
  if (live) {
    // the LANES threads of a token are all live or all not, so the shuffles
    // inside topk_lanes only read live threads
    const float* row = logits + (size_t)t * E;
    float bv[MK];
    int bi[MK];
    float den;
    float mx1 = 0.f;
    if constexpr (LANES == 1) topk_regs<NV, MK>(row, E, k, bv, bi, mx1, den);
    else topk_lanes<4, NV / 4, MK>(row, E, k, q, bv, bi, den);
    const float mx = bv[0];
    float sel[MK];
    float selsum = 0.f;
#pragma unroll
    for (int j = 0; j < MK; ++j) {
      sel[j] = j < k ? expf(bv[j] - mx) : 0.f;
      selsum += sel[j];
    }
#pragma unroll
    for (int j = 0; j < MK; ++j) {
      if (j < k) {
        my_ids[j] = bi[j];
        if (j % LANES == q) {
          const float w = renorm ? sel[j] / selsum : sel[j] / den;
          ids[(size_t)t * k + j] = bi[j];
          topw[(size_t)t * k + j] = w;
          slot_w[(size_t)t * slots + j] = w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      if (j >= k && j < slots) {
        my_ids[j] = E + (j - k);
        if (j % LANES == q) slot_w[(size_t)t * slots + j] = 1.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < MS; ++j)
      if (j < slots && j % LANES == q) atomicOr(&bits[my_ids[j]][tl >> 5], 1u << (tl & 31));
  }
  __syncthreads();

  // stable rank of each slot among earlier tokens of this block with the same expert
  if (live) {
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      if (j < slots && j % LANES == q) {
        const uint32_t* brow = bits[my_ids[j]];
        int c = 0;
        for (int w = 0; w < (tl >> 5); ++w) c += __popc(brow[w]);
        c += __popc(brow[tl >> 5] & ((1u << (tl & 31)) - 1u));
        rank[j] = c;
      }
    }
  }
  int count = 0;
  if (tid < ET) {
    for (int w = 0; w < kBitWords; ++w) count += __popc(bits[tid][w]);
  }
  if (gridDim.x == 1) {
    // one wave scans the expert counts with lane shuffles (up to 64 experts
    // straight from the counting threads, up to 256 four per lane through
    // LDS); scan_lds ends up holding each expert's offset
    if (ET <= 64) {
      if (tid < 64) {
        const int v = tid < ET ? count : 0;
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(incl, o);
          if (tid >= o) incl += u;
        }
        if (tid < ET) {
          scan_lds[tid] = incl - v;
          offsets[tid] = incl - v;
        }
        if (tid == 63) offsets[ET] = incl;
      }
      __syncthreads();
    } else {
      if (tid < ET) scan_lds[tid] = count;
      __syncthreads();
      if (tid < 64) {
        int c[4], lsum = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * tid + u;
          c[u] = e < ET ? scan_lds[e] : 0;
          lsum += c[u];
        }
        int incl = lsum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(incl, o);
          if (tid >= o) incl += v;
        }
        int run = incl - lsum;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * tid + u;
          if (e < ET) {
            scan_lds[e] = run;
            offsets[e] = run;
          }
          run += c[u];
        }
        if (tid == 63) offsets[ET] = incl;
      }
      __syncthreads();
    }
    if (live) {
#pragma unroll
      for (int j = 0; j < MS; ++j) {
        if (j < slots && j % LANES == q) {
          const int s = t * slots + j;
          const int pos = scan_lds[my_ids[j]] + rank[j];
          sorted_pairs[pos] = s;
          pair_pos[s] = pos;
        }
      }
    }
  } else {
    if (tid < ET) block_counts[(size_t)blockIdx.x * ET + tid] = count;
    if (live) {
#pragma unroll
      for (int j = 0; j < MS; ++j)
        if (j < slots && j % LANES == q) pair_pos[t * slots + j] = rank[j];
    }
  }
}

__global__ void __launch_bounds__(kRouteBlock)
route_scan(int nblocks, int ET, int32_t* __restrict__ block_counts, int32_t* __restrict__ offsets) {
  __shared__ int scan_lds[kRouteBlock];
  const int tid = threadIdx.x;
  int run = 0;
  if (tid < ET) {
    for (int b = 0; b < nblocks; ++b) {
      const int c = block_counts[(size_t)b * ET + tid];
      block_counts[(size_t)b * ET + tid] = run;   // becomes the block's base
      run += c;
    }
  }
  int total;
  const int off = block_exclusive_scan(tid < ET ? run : 0, scan_lds, &total);
  if (tid < ET) offsets[tid] = off;
  if (tid == 0) offsets[ET] = total;
}

__global__ void __launch_bounds__(kRouteBlock)
route_scatter(int T, int E, int k, int S, const int32_t* __restrict__ ids,
              const int32_t* __restrict__ block_base, const int32_t* __restrict__ offsets,
              int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
  const int t = blockIdx.x * kRouteBlock + threadIdx.x;
  if (t >= T) return;
  const int ET = E + S, slots = k + S;
  for (int j = 0; j < slots; ++j) {
    const int e = slot_expert(ids + (size_t)t * k, j, k, E);
    const int s = t * slots + j;
    const int pos = offsets[e] + block_base[(size_t)blockIdx.x * ET + e] + pair_pos[s];
    sorted_pairs[pos] = s;
    pair_pos[s] = pos;
  }
}

// Wide rows (more than 16 experts), up to 256 tokens: two launches that
// spread the selection over many compute units instead of one block.
//
// route_topk_wave: one wave per token.  Lane l holds experts l + 64 u
// (u < NV); the row maximum and the softmax denominator are butterfly
// reductions (every lane ends with the same value); each of the k picks is a
// wave arg-max over (logit, lower expert id on ties) of the lanes' best
// remaining expert, the owning lane then marks it taken.  Lane j < k writes
// pick j's id and weight; lanes k .. k+S-1 the shared slots' weight 1.
template <int NV>
__global__ void __launch_bounds__(256)
route_topk_wave(const float* __restrict__ logits, int T, int E, int k, int S, int renorm,
                int32_t* __restrict__ ids, float* __restrict__ topw, float* __restrict__ slot_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                       // the whole wave
  const int slots = k + S;
  const float* row = logits + (size_t)t * E;
  float v[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) v[u] = lane + 64 * u < E ? row[lane + 64 * u] : -INFINITY;
  float mx = v[0];
#pragma unroll
  for (int u = 1; u < NV; ++u) mx = fmaxf(mx, v[u]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float den = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (lane + 64 * u < E) den += expf(v[u] - mx);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  uint32_t taken = 0;
  float bsel[kMaxK];
  int isel[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    bsel[j] = -INFINITY;
    isel[j] = 0;
    if (j < k) {
      float bv = -INFINITY;
      int bi = 1 << 30;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = lane + 64 * u;
        if (e < E && !((taken >> u) & 1u) && (bi == (1 << 30) || v[u] > bv)) {
          bv = v[u];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      bsel[j] = bv;
      isel[j] = bi;
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
  }
  float sel[kMaxK], selsum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    sel[j] = j < k ? expf(bsel[j] - mx) : 0.f;
    selsum += sel[j];
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k && lane == j) {
      const float w = renorm ? sel[j] / selsum : sel[j] / den;
      ids[(size_t)t * k + j] = isel[j];
      topw[(size_t)t * k + j] = w;
      slot_w[(size_t)t * slots + j] = w;
    }
  }
  if (lane >= k && lane < slots) slot_w[(size_t)t * slots + lane] = 1.0f;
}

// route_sort_block: one block, up to 256 tokens.  Each slot's expert (from
// the picks, or the shared experts) sets its token's bit in an LDS bitmap
// per expert; the expert counts are scanned by one wave into the offsets;
// a slot's position is its expert's offset plus the number of earlier
// tokens with that expert (popcounts of the bitmap), which keeps pairs in
// slot order within an expert.
__global__ void __launch_bounds__(1024)
route_sort_block(const int32_t* __restrict__ ids, int T, int E, int k, int S, int32_t* __restrict__ sorted_pairs,
                 int32_t* __restrict__ pair_pos, int32_t* __restrict__ offsets) {
  __shared__ uint32_t bits[kMaxExperts][kBitWords];
  __shared__ int scan_lds[kMaxExperts];
  const int tid = threadIdx.x;
  const int ET = E + S, slots = k + S, P = T * slots;
  for (int x = tid; x < ET * kBitWords; x += 1024) (&bits[0][0])[x] = 0u;
  __syncthreads();
  constexpr int kPer = kRouteBlock * kMaxSlots / 1024;   // slots per thread, at most
  int ex[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int s = tid + 1024 * u;
    ex[u] = 0;
    if (s < P) {
      const int t = s / slots, j = s - t * slots;
      ex[u] = j < k ? ids[(size_t)t * k + j] : E + (j - k);
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int s = tid + 1024 * u;
    if (s < P) {
      const int t = s / slots;
      atomicOr(&bits[ex[u]][t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  // one wave scans the expert counts, four experts per lane
  if (tid < 64) {
    int c[4], lsum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      c[u] = 0;
      if (e < ET)
        for (int w = 0; w < kBitWords; ++w) c[u] += __popc(bits[e][w]);
      lsum += c[u];
    }
    int incl = lsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    int run = incl - lsum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      if (e < ET) {
        scan_lds[e] = run;
        offsets[e] = run;
      }
      run += c[u];
    }
    if (tid == 63) offsets[ET] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int s = tid + 1024 * u;
    if (s < P) {
      const int t = s / slots;
      const uint32_t* brow = bits[ex[u]];
      int r = 0;
      for (int w = 0; w < (t >> 5); ++w) r += __popc(brow[w]);
      r += __popc(brow[t >> 5] & ((1u << (t & 31)) - 1u));
      const int pos = scan_lds[ex[u]] + r;
      sorted_pairs[pos] = s;
      pair_pos[s] = pos;
    }
  }
}

int32_t launch_route(const float* logits, int T, int E, int k, int S, int renorm,
                     int32_t* ids, float* w, float* slot_w, int32_t* sorted_pairs,
                     int32_t* pair_pos, int32_t* offsets, void* ws, hipStream_t st) {
  const int nblocks = (T + kRouteBlock - 1) / kRouteBlock;
  int32_t* counts = (int32_t*)ws;
  if (E > 16 && T <= kRouteBlock) {
    // wide rows, one token block: the selection on one wave per token over
    // many compute units, then the sort in one block (C4: 23.6 us in one
    // block before)
    const dim3 g((T + 3) / 4);
    if (E <= 64) hipLaunchKernelGGL(route_topk_wave<1>, g, dim3(256), 0, st, logits, T, E, k, S, renorm, ids, w, slot_w);
    else if (E <= 128) hipLaunchKernelGGL(route_topk_wave<2>, g, dim3(256), 0, st, logits, T, E, k, S, renorm, ids, w, slot_w);
    else hipLaunchKernelGGL(route_topk_wave<4>, g, dim3(256), 0, st, logits, T, E, k, S, renorm, ids, w, slot_w);
    int32_t rc = hip_status(hipGetLastError(), "route_topk_wave launch");
    if (rc != MILO_OK) return rc;
    hipLaunchKernelGGL(route_sort_block, dim3(1), dim3(1024), 0, st, ids, T, E, k, S, sorted_pairs, pair_pos, offsets);
    return hip_status(hipGetLastError(), "route_sort_block launch");
  }
  // one thread per token up to 16 experts, four above (shorter selection chains)
#define MILO_ROUTE_LAUNCH(L, NV, MK, MS)                                                                             \
  hipLaunchKernelGGL((route_topk<L, NV, MK, MS>), dim3(nblocks), dim3(L * kRouteBlock), 0, st, logits, T, E, k, S, \
                     renorm, ids, w, slot_w, sorted_pairs, pair_pos, offsets, counts)
  const bool narrow = k <= 2 && k + S <= 4;   // top-1/top-2 with few shared experts
  if (E <= 8 && narrow) MILO_ROUTE_LAUNCH(1, 8, 2, 4);
  else if (E <= 8) MILO_ROUTE_LAUNCH(1, 8, kMaxK, kMaxSlots);
  else if (E <= 16 && narrow) MILO_ROUTE_LAUNCH(1, 16, 2, 4);
  else if (E <= 16) MILO_ROUTE_LAUNCH(1, 16, kMaxK, kMaxSlots);
  else if (E <= 32) MILO_ROUTE_LAUNCH(4, 32, kMaxK, kMaxSlots);
  else if (E <= 64) MILO_ROUTE_LAUNCH(4, 64, kMaxK, kMaxSlots);
  else if (E <= 128) MILO_ROUTE_LAUNCH(4, 128, kMaxK, kMaxSlots);
  else MILO_ROUTE_LAUNCH(4, 256, kMaxK, kMaxSlots);
#undef MILO_ROUTE_LAUNCH
  int32_t rc = hip_status(hipGetLastError(), "route_topk launch");
  if (rc != MILO_OK || nblocks == 1) return rc;
  hipLaunchKernelGGL(route_scan, dim3(1), dim3(kRouteBlock), 0, st, nblocks, E + S, counts, offsets);
  rc = hip_status(hipGetLastError(), "route_scan launch");
  if (rc != MILO_OK) return rc;
  hipLaunchKernelGGL(route_scatter, dim3(nblocks), dim3(kRouteBlock), 0, st, T, E, k, S, ids,
                     counts, offsets, sorted_pairs, pair_pos);
  return hip_status(hipGetLastError(), "route_scatter launch");
}

}  // namespace milo
