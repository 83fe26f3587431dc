// Small-M (decode) path of the routed W3A16 + low-rank grouped GEMM.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up).  MiLo Kernel: an int3 x fp16
// GEMM with the dequantization fused into the kernel (no separate dequantized
// copy of the weights in memory), and asynchronous global loads to hide
// memory latency.  MiLo Algorithm: W_out = W_quant + U V.
//
// At decode an expert sees a handful of rows and the layer is a stream of
// packed weights.  Work items are (expert, 64-row n-tile, K split) over the
// experts with rows; a persistent grid of blocks takes items round robin.
// An item covers MP 16-row m-tiles of the expert's rows (MP = 1: up to 16
// rows, MP = 2: up to 32).  The four waves of a block split the item: wave w
// takes m-tile w / KW and every KW-th 128-wide K block from w % KW on
// (KW = 4 / MP), so every wave holds one m-tile's registers and the waves of
// different m-tiles read the same code tiles at about the same time (the
// second read is served by the caches).  Each wave runs one continuous stream
// of K blocks across all of its items, with the loads of the next DEPTH-1 K
// blocks in flight in a register ring while the current one is consumed, so
// item boundaries do not drain the pipeline.  Every load in the stream is issued unconditionally
// (past the end a wave re-reads its last block), so the compiler's wait counts
// stay exact.
//
// Dequantization is folded out of the inner product.  One v_and_or_b32 turns
// a pair of int3 codes into two exact fp16 values off + q (off = 64 or 8);
// per 64-wide group the matrix cores compute P = sum_k x_k (off_k + q_k) from
// an accumulator preset to -(sum_k x_k off_k) - z (sum_k x_k), so that
// P = sum_k x_k (q_k - z), and y += s P in fp32.  The two activation sums are
// themselves matrix-core products of the activation fragments with constant
// fragments (all ones, and the offsets), so no weight is ever rounded to fp16
// and no extra data is loaded.  The expert's rows are the A operand (16 per
// m-tile; rows past the expert's count are zero), the codes the B operand.
//
// Item end: the low-rank term (x V^T) U^T of each m-tile is added by the
// waves of that m-tile, split by weight family and 32-rank step (their T and
// U fragments were loaded when the item started; int3 U tiles are extracted
// and dequantized here),
// the waves are summed in LDS in wave order, and the epilogue stores fp16
// (NONE / SWIGLU) or scales by the pair's route weight and scatters fp32
// (ROUTE_SCALE).  With
// several K splits each split stores its sum and gemm_decode_reduce adds the
// splits in split order (no cross-block synchronisation inside a kernel).
#include "gemm_common.hpp"

namespace milo {

constexpr int kMaxE = 256;

template <int WF, int WMT>
struct Stage {
  u32x4 q[WF][3];    // three planes of the 64 x 128 code tile, per family of the wave
  u32x4 z[WF][2];    // eight scale/zero words of this lane's rows
  f16x8 x[WMT][4];   // activation fragments of the four 32-wide K steps, per m-tile of the wave
};

struct Item {
  int e, nt, ks, base, M, kbA, kbB;
};

struct Cursor {
  int it;            // item index
  int kb;            // K block of this wave in the item
  bool valid;
  Item item;
};

// Work list entries: (expert, row chunk) as e << 8 | chunk.
constexpr int kMaxAct = 1024;

struct DecShared {
  int off[kMaxE + 1];
  int act[kMaxAct];
  int rank[2][kMaxE];
  int nact;
  int over;   // some expert has more rows than this launch handles
  int all;    // the chunk list overflowed: every expert counts as over
};

// Output rows of experts with more rows than the small-M path takes, when no
// other launch of the call covers them (the caller's row bound was wrong):
// they are set to NaN instead of being left unwritten.  Grid-strided over
// the rows x N outputs of each such expert.
template <int EPI>
__device__ void poison_over_rows(const GemmArgs& a, const DecShared& sh) {
  const int stride = gridDim.x * blockDim.x;
  for (int e = 0; e < a.num_experts; ++e) {
    const int base = sh.off[e], M = sh.off[e + 1] - base;
    if (M <= a.m_hi && !sh.all) continue;
    const int64_t n = (int64_t)M * a.N;
    for (int64_t o = blockIdx.x * blockDim.x + threadIdx.x; o < n; o += stride) {
      const int row = (int)(o / a.N), col = (int)(o - (int64_t)row * a.N);
      const int i = base + row;
      if (EPI == MILO_EPI_ROUTE_SCALE) ((float*)a.y)[(size_t)a.sorted_pairs[i] * a.N + col] = __builtin_nanf("");
      else ((uint16_t*)a.y)[(size_t)i * a.N + col] = 0x7E00u;   // fp16 quiet NaN
    }
  }
}


// Wave split of an item.  Default (FS = false): wave w takes m-tile w / KW
// and every KW-th K block from w % KW (KW = 4 / MP), with every weight family.
// Family split (FS = true, two m-tiles and two families): wave w takes family
// w % 2 and every second K block from w / 2, with both m-tiles, so each code
// is extracted once per item instead of once per m-tile.
template <int MP, int NW, int EPI, bool FS>
struct Dec {
  static constexpr int KW = FS ? 2 : 4 / MP;   // waves that split the K blocks of one output set
  static constexpr int WF = FS ? 1 : NW;       // weight families per wave
  static constexpr int WMT = FS ? MP : 1;      // m-tiles per wave
  const GemmArgs& a;
  const DecShared& sh;
  int lane, wave, kw, mtile, fam, total;
  CodeConsts kc;

  __device__ __forceinline__ Dec(const GemmArgs& a_, const DecShared& sh_, int total_)
      : a(a_), sh(sh_), lane(threadIdx.x & 63), wave(threadIdx.x >> 6),
        kw(__builtin_amdgcn_readfirstlane(FS ? (threadIdx.x >> 6) / 2 : (threadIdx.x >> 6) % KW)),
        mtile(__builtin_amdgcn_readfirstlane(FS ? 0 : (threadIdx.x >> 6) / KW)),
        fam(__builtin_amdgcn_readfirstlane(FS ? (threadIdx.x >> 6) % 2 : 0)), total(total_),
        kc(make_code_consts()) {}

  __device__ __forceinline__ void enter(Cursor& c, int it) const {
    if (it >= total) {
      c.valid = false;          // keep the last item and K block for dummy loads
      return;
    }
    // all item fields are wave-uniform: keep them in scalar registers
    const int per_e = a.n_tiles * a.ksplit;
    const int ai = it / per_e;
    const int r = it - ai * per_e;
    Item& m = c.item;
    const int ent = __builtin_amdgcn_readfirstlane(sh.act[ai]);
    m.e = ent >> 8;
    m.nt = r / a.ksplit;
    m.ks = r - m.nt * a.ksplit;
    m.base = __builtin_amdgcn_readfirstlane(sh.off[m.e]) + (ent & 255) * a.m_hi;
    const int rest = __builtin_amdgcn_readfirstlane(sh.off[m.e + 1]) - m.base;
    m.M = rest < a.m_hi ? rest : a.m_hi;
    m.kbA = (int)((int64_t)a.kblocks * m.ks / a.ksplit);
    m.kbB = (int)((int64_t)a.kblocks * (m.ks + 1) / a.ksplit);
    c.it = it;
    c.kb = m.kbA + kw;
    c.valid = true;
  }
  __device__ __forceinline__ bool last(const Cursor& c) const { return c.kb + KW >= c.item.kbB; }
  __device__ __forceinline__ void next(Cursor& c) const {
    if (!c.valid) return;
    if (!last(c)) c.kb += KW;
    else enter(c, c.it + gridDim.x);
  }

  // A wave whose first K block lies past the item's range (K splits of fewer
  // than four blocks) gets one null element: real codes of the item's first
  // block with zero activations, which adds exactly zero.
  __device__ __forceinline__ void load(Stage<WF, WMT>& S, const Cursor& c) const {
    const Item& m = c.item;
    const bool live = c.kb < m.kbB;
    const int kb = live ? c.kb : m.kbA;
#pragma unroll
    for (int fl = 0; fl < WF; ++fl) {
      const int f = FS ? fam : fl;
      const uint32_t* tp = a.packed[f] + m.e * a.words_per_expert +
                           ((size_t)m.nt * a.kblocks + kb) * kTileWords + 4 * lane;
      // codes are read once per launch: non-temporal loads (measured: C2
      // gate/up 85.2 -> 83.7 us)
      S.q[fl][0] = __builtin_nontemporal_load((const u32x4*)(tp));
      S.q[fl][1] = __builtin_nontemporal_load((const u32x4*)(tp + 256));
      S.q[fl][2] = __builtin_nontemporal_load((const u32x4*)(tp + 512));
      const uint32_t* sp = a.sz[f] + m.e * a.sz_per_expert +
                           ((size_t)m.nt * a.kblocks + kb) * kTileSzWords + 8 * (lane & 15);
      S.z[fl][0] = *(const u32x4*)(sp);
      S.z[fl][1] = *(const u32x4*)(sp + 4);
    }
#pragma unroll
    for (int mt = 0; mt < WMT; ++mt) {
      const int row = (mtile + mt) * 16 + (lane & 15);
      const bool ok = live && row < m.M;
      const uint16_t* xp =
          a.x + (size_t)(m.base + (row < m.M ? row : 0)) * a.K + (size_t)kb * kTileK + 8 * (lane >> 4);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 v = *(const f16x8*)(xp + 32 * s);
        S.x[mt][s] = ok ? v : f16x8{};
      }
    }
  }

  __device__ __forceinline__ void consume(const Stage<WF, WMT>& S, f32x4 (&acc)[WF][WMT][4]) const {
    const f16x8 one = ones_frag();
    // activation sums per group: xs = sum x, xo = sum x * off (rows of this lane)
    f32x4 xs[WMT][2], xo[WMT][2];
#pragma unroll
    for (int mt = 0; mt < WMT; ++mt)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        xs[mt][g] = mfma16x16x32(S.x[mt][2 * g], one, zero);
        xs[mt][g] = mfma16x16x32(S.x[mt][2 * g + 1], one, xs[mt][g]);
        xo[mt][g] = mfma16x16x32(S.x[mt][2 * g], offset_frag(2 * g), zero);
        xo[mt][g] = mfma16x16x32(S.x[mt][2 * g + 1], offset_frag(2 * g + 1), xo[mt][g]);
      }
#pragma unroll
    for (int f = 0; f < WF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h[16];
        extract_triplet(S.q[f][0][i], S.q[f][1][i], S.q[f][2][i], h, kc);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int idx = 2 * i + g;
          const uint32_t w = idx < 4 ? S.z[f][0][idx] : S.z[f][1][idx - 4];
          const float sc = half_bits_to_float(w & 0xFFFFu);
          const float zp = half_bits_to_float(w >> 16);
#pragma unroll
          for (int mt = 0; mt < WMT; ++mt) {
            f32x4 p;
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = __builtin_fmaf(-zp, xs[mt][g][r], -xo[mt][g][r]);
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
              const int step = 2 * g + ss;
              const u32x4 u = {h[4 * step], h[4 * step + 1], h[4 * step + 2], h[4 * step + 3]};
              p = mfma16x16x32(S.x[mt][step], __builtin_bit_cast(f16x8, u), p);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[f][mt][i][r] = __builtin_fmaf(sc, p[r], acc[f][mt][i][r]);
          }
        }
      }
  }
};

// U operand of the low-rank term of one item (the NS rank steps of 32 that
// this wave adds): fp16 fragments (64 n rows x 32 ranks per step), or with
// int3 factors the lane's triplet of each 32-rank U tile plus the scale/zero
// words of its four rows (dequantized at the item's end).
template <bool LRQ, int NS>
struct LateU {
  f16x8 u[4][NS];
};
template <int NS>
struct LateU<true, NS> {
  uint32_t q[NS][3];
  u32x4 sz;
};

// Per-item values loaded when an item starts and used at its end.
template <int MP, bool LRQ, int NS, int WMT>
struct ItemLate {
  f16x8 t[WMT][NS];   // low-rank T fragments (rows of each m-tile of the wave x 32 ranks)
  LateU<LRQ, NS> lu;  // U operand of this wave's family
  int32_t sp[MP * 4]; // ROUTE_SCALE: slot index of each output row of this thread
  float pw[MP * 4];   // ROUTE_SCALE: route weight of those rows
};

template <int MP, int NW, int EPI, int DEPTH, bool LRQ, bool FS = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_decode_kernel(GemmArgs a) {
  using DecT = Dec<MP, NW, EPI, FS>;
  constexpr int KW = DecT::KW;
  constexpr int WF = DecT::WF, WMT = DecT::WMT;
  __shared__ DecShared sh;
  constexpr int kTile = 16 * 64;           // outputs of one m-tile per family
  constexpr int kOut = MP * kTile;         // outputs per family per item
  constexpr int kPer = kOut / 256;         // per thread
  // wave partials: [wave][family of the wave][m-tile of the wave] (WF x WMT = NW or MP tiles)
  __shared__ float red[4][WF * WMT][kTile];

  // ---- experts with rows for this path, and their ranks
  for (int e = threadIdx.x; e <= a.num_experts; e += 256) sh.off[e] = a.offsets[e];
  for (int e = threadIdx.x; e < a.num_experts; e += 256) {
    sh.rank[0][e] = a.rp ? a.rank[0][e] : 0;
    sh.rank[1][e] = a.rp ? a.rank[NW - 1][e] : 0;
  }
  __syncthreads();
  // the work list, built by the first wave: lane l takes experts 4l .. 4l+3,
  // counts their entries (one per expert in [m_lo, m_hi] rows, or with
  // dec_chunk one per m_hi-row chunk of every expert with rows), and a lane
  // scan places them in expert order.  A list past kMaxAct entries (possible
  // only when the caller's row bound was wrong) is dropped whole: every
  // expert then counts as over.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int cnt[4], tot = 0, over = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * lane + c;
      const int M = e < a.num_experts ? sh.off[e + 1] - sh.off[e] : 0;
      int n;
      if (a.dec_chunk) {
        n = M > 0 ? (M + a.m_hi - 1) / a.m_hi : 0;
        over |= n > 256;                 // chunk index past 8 bits
      } else {
        n = (M >= a.m_lo && M <= a.m_hi) ? 1 : 0;
        over |= M > a.m_hi;
      }
      cnt[c] = n;
      tot += n;
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63);
    const int any_over = __any(over);
    const bool fits = total <= kMaxAct && !(a.dec_chunk && any_over);
    if (fits) {
      int idx = incl - tot;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        for (int j = 0; j < cnt[c]; ++j) sh.act[idx++] = ((4 * lane + c) << 8) | j;
    }
    if (lane == 0) {
      sh.nact = fits ? total : 0;
      sh.all = fits ? 0 : 1;
      sh.over = (any_over || !fits) ? 1 : 0;
    }
  }
  __syncthreads();
  if (a.poison_over && sh.over) poison_over_rows<EPI>(a, sh);
  const int total = __builtin_amdgcn_readfirstlane(sh.nact) * a.n_tiles * a.ksplit;
  if ((int)blockIdx.x >= total) return;

  DecT D(a, sh, total);
  const int lane = D.lane, wave = D.wave, kw = D.kw, mtile = D.mtile;
  const int RW = a.n_w * a.rp;
  // low-rank work of this wave: family lrf, rank steps (32 ranks each)
  // s2_0 + l LRW for l < NS, so the waves that share an output set share its
  // item-end work (steps past the padded rank are skipped).  Default split:
  // family kw mod NW, steps from kw / NW in strides of KW / NW.  Family split:
  // the wave's own family, steps from kw in strides of KW (one step each for
  // ranks up to 64).
  constexpr int LRW = FS ? KW : KW / NW;
  constexpr int NS = FS ? 1 : (LRW >= 2 ? 1 : 2);
  const int lrf = FS ? D.fam : kw % NW;
  const int s2_0 = FS ? kw : kw / NW;

  f32x4 acc[WF][WMT][4];
#pragma unroll
  for (int f = 0; f < WF; ++f)
#pragma unroll
    for (int mt = 0; mt < WMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // item-start loads: low-rank fragments (every wave loads, waves that add no
  // low-rank term ignore them) and the epilogue's row metadata.  Addresses are
  // clamped to valid memory and masked values replaced, so every load is issued.
  ItemLate<MP, LRQ, NS, WMT> late;
  auto load_late = [&](const Item& m) {
    if (a.rp > 0) {
      const int rk = sh.rank[lrf][m.e];
#pragma unroll
      for (int l = 0; l < NS; ++l) {
        const int s2 = s2_0 + l * LRW;
        const int j0 = 32 * s2 + 8 * (lane >> 4);
        const bool jok = j0 < rk;
        const int jc = jok ? j0 : 0;
#pragma unroll
        for (int mt = 0; mt < WMT; ++mt) {
          const int row = (mtile + mt) * 16 + (lane & 15);
          const bool ok = jok && row < m.M;
          const f16x8 v =
              *(const f16x8*)(a.T + (size_t)(m.base + (row < m.M ? row : 0)) * RW + lrf * a.rp + jc);
          late.t[mt][l] = ok ? v : f16x8{};    // ranks >= rank: zero, so U's padding adds nothing
        }
        if constexpr (LRQ) {
          // 32-rank tile s2 if the expert has ranks there, else tile 0 (valid memory, unused)
          const int jt = 32 * s2 < rk ? s2 : 0;
          const uint32_t* up = a.Uq[lrf] + m.e * a.uq_per_expert +
                               ((size_t)m.nt * (a.rp / 32) + jt) * 192 + lane;
          late.lu.q[l][0] = up[0];
          late.lu.q[l][1] = up[64];
          late.lu.q[l][2] = up[128];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = m.nt * kTileRows + 16 * i + (lane & 15);
            const f16x8 u = *(const f16x8*)(a.U[lrf] + ((size_t)m.e * a.N + n) * a.max_rank + jc);
            late.lu.u[i][l] = jok ? u : f16x8{};
          }
        }
      }
      if constexpr (LRQ)
        late.lu.sz = *(const u32x4*)(a.Usz[lrf] + (size_t)m.e * a.N + m.nt * kTileRows + 4 * (lane & 15));
    }
    if (EPI == MILO_EPI_ROUTE_SCALE) {
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        const int row = (threadIdx.x + 256 * c) >> 6;
        const int i = m.base + (row < m.M ? row : 0);
        late.sp[c] = a.sorted_pairs[i];
        late.pw[c] = a.pw[i];
      }
    }
  };

  auto finish_item = [&](const Item& m) {
    // low-rank term of family lrf, rank steps s2_0 + l LRW, for this wave's
    // m-tiles (added once: by the first K split)
    if (a.rp > 0 && m.ks == 0) {
#pragma unroll
      for (int l = 0; l < NS; ++l) {
        const int s2 = s2_0 + l * LRW;
        if (32 * s2 >= a.rp) break;
        if constexpr (LRQ) {
          uint32_t h[16];
          extract_triplet(late.lu.q[l][0], late.lu.q[l][1], late.lu.q[l][2], h, D.kc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x8 ub = dequant_step(h, i, group_const(late.lu.sz[i]));
#pragma unroll
            for (int f = 0; f < WF; ++f)
#pragma unroll
              for (int mt = 0; mt < WMT; ++mt)
                if (FS || f == lrf) acc[f][mt][i] = mfma16x16x32(late.t[mt][l], ub, acc[f][mt][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int f = 0; f < WF; ++f)
#pragma unroll
              for (int mt = 0; mt < WMT; ++mt)
                if (FS || f == lrf)
                  acc[f][mt][i] = mfma16x16x32(late.t[mt][l], late.lu.u[i][l], acc[f][mt][i]);
        }
      }
    }
    __syncthreads();   // previous item's readers of red are done
#pragma unroll
    for (int f = 0; f < WF; ++f)
#pragma unroll
      for (int mt = 0; mt < WMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 4 * (lane >> 4) + r, n = 16 * i + (lane & 15);
            red[wave][f * WMT + mt][row * 64 + n] = acc[f][mt][i][r];
          }
          acc[f][mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    __syncthreads();
    // the item's outputs per family, the K-split waves added in wave order:
    // default split, waves mt KW .. mt KW + KW - 1 hold m-tile mt (every
    // family); family split, waves 2 kw + f hold family f (every m-tile)
    float res[NW][kPer];
#pragma unroll
    for (int f = 0; f < NW; ++f)
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        const int o = threadIdx.x + 256 * c;
        const int mt = o / kTile, ol = o - mt * kTile;   // m-tile and offset within it
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < KW; ++w) v += FS ? red[2 * w + f][mt][ol] : red[mt * KW + w][f][ol];
        res[f][c] = v;
      }
    if (a.ksplit > 1) {
      float* mine = a.part + (((size_t)m.ks * a.num_experts + m.e) * a.n_tiles + m.nt) * (NW * kOut);
#pragma unroll
      for (int f = 0; f < NW; ++f)
#pragma unroll
        for (int c = 0; c < kPer; ++c) mine[f * kOut + threadIdx.x + 256 * c] = res[f][c];
      return;
    }
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int o = threadIdx.x + 256 * c;
      const int row = o >> 6, n = o & 63;
      if (row >= m.M) continue;
      const int col = m.nt * kTileRows + n;
      if (EPI == MILO_EPI_ROUTE_SCALE) {
        ((float*)a.y)[(size_t)late.sp[c] * a.N + col] = res[0][c] * late.pw[c];
      } else {
        float v = res[0][c];
        if (EPI == MILO_EPI_SWIGLU) v = silu(v) * res[NW - 1][c];
        ((uint16_t*)a.y)[(size_t)(m.base + row) * a.N + col] = float_to_half_bits(v);
      }
    }
  };

  Cursor pf, cs;
  D.enter(pf, blockIdx.x);
  cs = pf;
  load_late(cs.item);
  Stage<WF, WMT> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) {
    D.load(ring[d], pf);
    D.next(pf);
  }
  while (cs.valid) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (cs.valid) {
        D.load(ring[(d + DEPTH - 1) % DEPTH], pf);
        D.next(pf);
        D.consume(ring[d], acc);
        if (D.last(cs)) {
          finish_item(cs.item);
          D.next(cs);
          if (cs.valid) load_late(cs.item);
        } else {
          D.next(cs);
        }
      }
    }
  }
}

template <int MP, int NW, int EPI>
static void launch_one(const GemmArgs& a, int blocks, int num_experts, hipStream_t st) {
  constexpr int depth = NW == 1 ? 3 : 2;
  // two m-tiles of gate/up: the family split (each code extracted once)
  constexpr bool fs = MP == 2 && NW == 2;
  if (a.lrq)
    hipLaunchKernelGGL((gemm_decode_kernel<MP, NW, EPI, depth, true, fs>), dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<MP, NW, EPI, depth, false, fs>), dim3(blocks), dim3(256), 0, st, a);
  if (a.ksplit > 1)
    hipLaunchKernelGGL((gemm_split_reduce<16 * MP, NW, EPI>), dim3(a.n_tiles, num_experts), dim3(256), 0,
                       st, a);
}

template <int MP>
static void launch_mt(const GemmArgs& a, int epi, int blocks, int num_experts, hipStream_t st) {
  switch (epi) {
    case MILO_EPI_SWIGLU: launch_one<MP, 2, MILO_EPI_SWIGLU>(a, blocks, num_experts, st); break;
    case MILO_EPI_ROUTE_SCALE: launch_one<MP, 1, MILO_EPI_ROUTE_SCALE>(a, blocks, num_experts, st); break;
    default: launch_one<MP, 1, MILO_EPI_NONE>(a, blocks, num_experts, st); break;
  }
}

int32_t launch_gemm_decode(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  if (p.dec_mt == 0) return MILO_OK;
  GemmArgs a = make_gemm_args(d, p, ws);
  a.part = (float*)(ws + p.off_dec_part);
  if (d->gather_div > 0) a.x = (const uint16_t*)(ws + p.off_xg);   // pair-ordered rows
  a.pw = (const float*)(ws + p.off_pw);
  a.m_lo = 1;
  a.m_hi = p.dec_max_rows;
  // without a tile launch the small-M launch takes every expert, the larger
  // ones in chunks of m_hi rows (split K indexes its partial sums by expert,
  // so it keeps the row range and NaN-fills experts above it instead)
  a.dec_chunk = (!p.pre_launch && p.dec_ksplit == 1) ? 1 : 0;
  a.poison_over = (!p.pre_launch && !a.dec_chunk) ? 1 : 0;
  switch (p.dec_mt) {
    case 1: launch_mt<1>(a, d->epilogue, p.dec_blocks, d->num_experts, st); break;
    case 2: launch_mt<2>(a, d->epilogue, p.dec_blocks, d->num_experts, st); break;
    default: set_error("internal: bad m-tile count %d", p.dec_mt); return MILO_ERR_ARG;
  }
  return hip_status(hipGetLastError(), "gemm_decode_kernel launch");
}

}  // namespace milo
