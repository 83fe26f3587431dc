// The C ABI of libmilo (declared in include/milo.h): argument validation,
// workspace planning and kernel dispatch.  Host code only; every check runs
// before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "gemm_common.hpp"

namespace milo {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MILO_OK;
  set_error("%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return MILO_ERR_HIP;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

#define MILO_FAIL(code, ...)   \
  do {                         \
    set_error(__VA_ARGS__);    \
    return (code);             \
  } while (0)

GemmArgs make_gemm_args(const milo_gemm_desc* d, const GemmPlan& p, char* ws) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.x = d->x;
  a.sorted_pairs = d->sorted_pairs;
  a.offsets = d->offsets;
  a.slot_w = d->slot_w;
  for (int f = 0; f < 2; ++f) {
    const milo_weights& w = d->w[f < d->n_w ? f : 0];
    a.packed[f] = w.packed;
    a.sz[f] = w.sz;
    a.U[f] = w.U;
    a.Uq[f] = w.Uq;
    a.Usz[f] = w.Usz;
    a.rank[f] = w.rank;
  }
  a.lrq = d->w[0].lr_format == MILO_LR_INT3 ? 1 : 0;
  a.uq_per_expert = d->max_rank ? milo_lr_u_words(d->N, d->max_rank) : 0;
  a.T = (const uint16_t*)(ws + p.off_t);
  a.y = d->y;
  a.words_per_expert = milo_packed_words(d->N, d->K);
  a.sz_per_expert = milo_sz_words(d->N, d->K);
  a.N = d->N;
  a.K = d->K;
  a.kblocks = p.kblocks;
  a.n_tiles = p.n_tiles;
  a.gather_div = d->gather_div;
  a.num_experts = d->num_experts;
  a.n_w = d->n_w;
  a.rp = p.rp;
  a.max_rank = d->max_rank;
  a.epilogue = d->epilogue;
  a.ksplit = p.dec_ksplit;
  a.dec_max_rows = p.dec_max_rows;
  a.pre_min_rows = p.pre_launch ? (p.dec_mt ? p.dec_max_rows : 0) : 0;
  a.x_bytes_32 = (uint64_t)d->x_rows * (uint64_t)d->K * 2u < (1ull << 32) ? 1 : 0;
  return a;
}

static int32_t validate_gemm(const milo_gemm_desc* d) {
  if (!d) MILO_FAIL(MILO_ERR_NULL, "desc is NULL");
  if (d->num_experts < 1 || d->num_experts > 256)
    MILO_FAIL(MILO_ERR_SHAPE, "num_experts=%d outside 1..256", d->num_experts);
  if (d->N <= 0 || d->K <= 0 || d->N > 65536 || d->K > 65536 || d->N % 64 || d->K % 128)
    MILO_FAIL(MILO_ERR_SHAPE, "N=%d K=%d: need N %% 64 == 0, K %% 128 == 0, both in 1..65536", d->N, d->K);
  if (d->max_rank < 0 || d->max_rank > kMaxRank || d->max_rank % 8)
    MILO_FAIL(MILO_ERR_RANK, "max_rank=%d: need 0..64, multiple of 8", d->max_rank);
  if (d->epilogue < MILO_EPI_NONE || d->epilogue > MILO_EPI_ROUTE_SCALE)
    MILO_FAIL(MILO_ERR_ARG, "unknown epilogue %d", d->epilogue);
  if (d->path < MILO_PATH_AUTO || d->path > MILO_PATH_PREFILL)
    MILO_FAIL(MILO_ERR_ARG, "unknown path %d", d->path);
  if ((d->epilogue == MILO_EPI_SWIGLU) != (d->n_w == 2) || (d->n_w != 1 && d->n_w != 2))
    MILO_FAIL(MILO_ERR_ARG, "n_w=%d does not match epilogue %d (SWIGLU needs 2, others 1)", d->n_w, d->epilogue);
  if (d->num_pairs < 0 || d->num_pairs > (1 << 20))
    MILO_FAIL(MILO_ERR_SHAPE, "num_pairs=%d outside 0..1048576", d->num_pairs);
  if (d->max_rows_per_expert < 0) MILO_FAIL(MILO_ERR_SHAPE, "max_rows_per_expert < 0");
  if (d->gather_div < 0) MILO_FAIL(MILO_ERR_SHAPE, "gather_div < 0");
  if (d->x_rows < 0) MILO_FAIL(MILO_ERR_SHAPE, "x_rows < 0");
  if (!d->x || !d->offsets || !d->y) MILO_FAIL(MILO_ERR_NULL, "x, offsets and y are required");
  if ((d->gather_div > 0 || d->epilogue == MILO_EPI_ROUTE_SCALE) && !d->sorted_pairs)
    MILO_FAIL(MILO_ERR_NULL, "sorted_pairs is required with gather_div > 0 or ROUTE_SCALE");
  if (d->epilogue == MILO_EPI_ROUTE_SCALE && (!d->slot_w || d->y_rows < 1))
    MILO_FAIL(MILO_ERR_NULL, "ROUTE_SCALE needs slot_w and y_rows >= 1");
  for (int f = 0; f < d->n_w; ++f) {
    const milo_weights& w = d->w[f];
    if (!w.packed || !w.sz) MILO_FAIL(MILO_ERR_NULL, "w[%d].packed / sz is NULL", f);
    if (w.lr_format != MILO_LR_FP16 && w.lr_format != MILO_LR_INT3)
      MILO_FAIL(MILO_ERR_ARG, "w[%d].lr_format=%d unknown", f, w.lr_format);
    if (w.lr_format != d->w[0].lr_format)
      MILO_FAIL(MILO_ERR_ARG, "both weight families need the same lr_format");
    if (d->max_rank > 0 && !w.rank) MILO_FAIL(MILO_ERR_NULL, "w[%d].rank is NULL with max_rank > 0", f);
    if (d->max_rank > 0 && w.lr_format == MILO_LR_FP16 && (!w.U || !w.V))
      MILO_FAIL(MILO_ERR_NULL, "w[%d].U / V is NULL with max_rank > 0", f);
    if (d->max_rank > 0 && w.lr_format == MILO_LR_INT3 && (!w.Uq || !w.Usz || !w.Vq || !w.Vsz))
      MILO_FAIL(MILO_ERR_NULL, "w[%d].Uq / Usz / Vq / Vsz is NULL with max_rank > 0 (int3 factors)", f);
    if (!aligned(w.packed, 16) || !aligned(w.sz, 16) || !aligned(w.U, 16) || !aligned(w.V, 16) ||
        !aligned(w.Uq, 16) || !aligned(w.Usz, 16) || !aligned(w.Vq, 16) || !aligned(w.Vsz, 16))
      MILO_FAIL(MILO_ERR_ALIGN, "w[%d] pointers must be 16-byte aligned", f);
    if (w.rank && !aligned(w.rank, 4)) MILO_FAIL(MILO_ERR_ALIGN, "w[%d].rank must be 4-byte aligned", f);
  }
  if (!aligned(d->x, 16) || !aligned(d->y, 16))
    MILO_FAIL(MILO_ERR_ALIGN, "x and y must be 16-byte aligned");
  if (!aligned(d->offsets, 4) || !aligned(d->sorted_pairs, 4) || !aligned(d->slot_w, 4))
    MILO_FAIL(MILO_ERR_ALIGN, "offsets, sorted_pairs, slot_w must be 4-byte aligned");
  return MILO_OK;
}

// Compute units of the current device (cached per device; 256, the MI355X
// count, if the runtime cannot tell, e.g. on a host without a GPU where only
// workspace sizes are queried).
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cached[dev] = cus;
  return cus;
}

int32_t plan_gemm(const milo_gemm_desc* d, GemmPlan* p) {
  memset(p, 0, sizeof *p);
  p->n_tiles = d->N / kTileRows;
  p->kblocks = d->K / kTileK;
  p->rp = d->max_rank == 0 ? 0 : (int)round_up((size_t)d->max_rank, 32);
  const int P = d->num_pairs;
  int rows_bound = d->max_rows_per_expert > 0 ? d->max_rows_per_expert : P;
  if (rows_bound > P) rows_bound = P;
  if (P == 0) return MILO_OK;  // nothing to do

  auto mt_for = [](int rows) { return rows <= 16 ? 1 : 2; };
  if (d->path == MILO_PATH_DECODE) {
    if (rows_bound > kDecodeMaxRows)
      MILO_FAIL(MILO_ERR_SHAPE, "decode path needs <= %d rows per expert (bound %d)", kDecodeMaxRows, rows_bound);
    p->dec_mt = mt_for(rows_bound);
  } else if (d->path == MILO_PATH_PREFILL) {
    p->dec_mt = 0;
    p->pre_launch = 1;
  } else if (rows_bound <= kDecodeMaxRows && !(rows_bound > 16 && (int64_t)d->N * d->K > kSmallMatrixElems)) {
    p->dec_mt = mt_for(rows_bound);
  } else if (rows_bound <= kDecodeMaxRows) {
    p->dec_mt = 1;
    p->dec_chunked = 1;
  } else if ((int64_t)d->N * d->K <= kSmallMatrixElems && P >= 16 * d->num_experts) {
    // small matrices, experts averaging 16 rows or more: the tile kernel for
    // every expert (measured: 1408 x 2048 experts, 31 rows on average,
    // 0.205 ms per layer with both paths -> 0.198 ms)
    p->dec_mt = 0;
    p->pre_launch = 1;
  } else if (rows_bound <= kDecodeChunkRows && P < 32 * d->num_experts &&
             (int64_t)d->N * d->K > kSmallMatrixElems) {
    // large matrices, experts averaging under 32 rows, none above
    // kDecodeChunkRows: the small-M kernel alone, experts above its rows in
    // chunks (each chunk streams the expert's weights again), instead of a
    // tile launch that mostly finds no expert (measured 4.6 us per empty
    // launch at 64 tokens over 8 experts).  16-row chunks on the one-m-tile
    // kernel: at 64 tokens over 8 experts (8..27 rows) as fast as 32-row
    // chunks on the two-m-tile gate/up kernel (gate/up 122 vs 124 us), which
    // reads the weights once but does twice the arithmetic per weight
    p->dec_mt = 1;
    p->dec_chunked = 1;
  } else if (P >= 64 * d->num_experts) {
    // experts averaging 64 rows or more: the tile kernel for every expert
    // (a small-M launch would find few experts or none; measured 4-5 us per
    // empty launch at 4096 tokens over 8 experts)
    p->dec_mt = 0;
    p->pre_launch = 1;
  } else {
    // both paths: the small-M kernel takes experts of up to 32 rows (two
    // m-tiles), or for small matrices only those of up to 16 rows, the tile
    // kernel the rest (measured: 1408 x 2048 experts 0.232 -> 0.206 ms per
    // layer; 14336 x 4096 experts at 8..22 rows 8.0 -> 11.6 ms for 32 layers)
    p->dec_mt = (int64_t)d->N * d->K <= kSmallMatrixElems ? 1 : 2;
    p->pre_launch = 1;
  }
  p->dec_max_rows = 16 * p->dec_mt;
  p->pre_bm = P >= 256 * d->num_experts ? 128 : 64;
  p->pre_tiles = (P + p->pre_bm - 1) / p->pre_bm + d->num_experts;
  p->pre_slots = 2 * device_cu_count();

  if (p->dec_mt) {
    // persistent grid: two blocks per compute unit (the kernel's register
    // budget allows two).  Split K only when it shortens the
    // busiest block's work (in items) to under 3/4 of the unsplit round: a
    // split costs a reduce launch, and e.g. 448 items take one round whether
    // split or not.  Keep at least four K blocks per split (one per wave).
    const int slots = 2 * device_cu_count();
    const int active = d->num_experts < P ? d->num_experts : P;
    const int items = active * p->n_tiles;
    int ks_max = p->kblocks / 4;
    if (ks_max < 1) ks_max = 1;
    int ks = 1;
    const double span1 = (double)((items + slots - 1) / slots);
    double best = span1;
    for (int k = 2; k <= ks_max && items < slots; ++k) {
      const double span = (double)((items * k + slots - 1) / slots) / k;
      if (span < 0.75 * span1 && span < best) {
        best = span;
        ks = k;
      }
    }
    p->dec_ksplit = p->dec_chunked ? 1 : ks;   // chunk entries have no split-K slot
    p->dec_blocks = items * ks < slots ? items * ks : slots;
  }
  p->lr_tiles = (P + 15) / 16 + d->num_experts;
  const int nrt = d->n_w * p->rp / 16;
  p->lr_tiles_per_block = rows_bound <= kDecodeMaxRows ? 1 : (nrt > 0 ? nrt : 1);
  p->lr_mt = 1;
  p->lr_ks = 1;
  if (p->rp > 0 && p->lr_tiles_per_block > 1 && d->w[0].lr_format == MILO_LR_FP16) {
    // fp16 prefill-form pre-pass.  Experts averaging 128 rows or more: the
    // 128-row tile kernel (all ranks per block), K split until the row tiles
    // (counted without partial tiles) fill about one block per CU, at least
    // four K blocks per chunk.  Otherwise 16-row tiles x groups of four rank
    // tiles, K split while they number fewer than kPrepassBlocks, keeping at
    // least one batch of loads (4 waves x 4 steps of 32) per chunk, and only
    // below 64 blocks.
    int ks;
    if (P >= 128 * d->num_experts) {
      p->lr_mt = kPrepassTileRows / 16;
      const int est = (P + kPrepassTileRows - 1) / kPrepassTileRows;
      ks = (256 + est - 1) / est;
      const int ks_max = (d->K / 128) / 4;
      if (ks > ks_max) ks = ks_max;
      if (ks < 1) ks = 1;
      const int per = (d->K / 128 + ks - 1) / ks;   // K blocks per chunk
      ks = (d->K / 128 + per - 1) / per;             // every chunk non-empty
    } else {
      p->lr_mt = 1;
      const int tpb = p->lr_tiles_per_block < 4 ? p->lr_tiles_per_block : 4;
      const int est = ((P + 15) / 16) * (nrt / tpb);
      // a split costs a reduce launch: it pays only where the unsplit grid
      // leaves most of the GPU idle (measured: 8 to 16 blocks gain three- to
      // fivefold, 128 to 256 blocks lose)
      ks = est < 64 ? (kPrepassBlocks + est - 1) / est : 1;
      const int ks_max = (d->K / 32) / 16;
      if (ks > ks_max) ks = ks_max;
      if (ks < 1) ks = 1;
      const int per = (d->K / 32 + ks - 1) / ks;     // K steps per chunk
      ks = (d->K / 32 + per - 1) / per;              // every chunk non-empty
    }
    p->lr_ks = ks < 1 ? 1 : ks;
  }

  size_t off = 0;
  p->off_t = off;
  off += round_up((size_t)P * d->n_w * p->rp * 2, 256);
  p->off_xg = off;
  if (p->dec_mt && d->gather_div > 0) off += round_up((size_t)P * d->K * 2, 256);
  p->off_pw = off;
  if (p->dec_mt && d->epilogue == MILO_EPI_ROUTE_SCALE) off += round_up((size_t)P * 4, 256);
  p->off_dec_part = off;
  if (p->dec_ksplit > 1)
    off += round_up((size_t)p->dec_ksplit * d->num_experts * p->n_tiles * d->n_w * p->dec_mt * 16 * 64 * 4, 256);
  p->off_tpart = off;
  if (p->lr_ks > 1) off += round_up((size_t)p->lr_ks * P * d->n_w * p->rp * 4, 256);
  p->total = off;
  return MILO_OK;
}

}  // namespace milo

using namespace milo;

extern "C" {

int32_t milo_abi_version(void) { return MILO_ABI_VERSION; }
int32_t milo_layout_version(void) { return MILO_LAYOUT_VERSION; }

const char* milo_status_string(int32_t s) {
  switch (s) {
    case MILO_OK: return "ok";
    case MILO_ERR_NULL: return "a required pointer is NULL";
    case MILO_ERR_SHAPE: return "a size violates the documented constraints";
    case MILO_ERR_ALIGN: return "a pointer is not aligned as documented";
    case MILO_ERR_RANK: return "compensator rank outside the supported range";
    case MILO_ERR_WORKSPACE: return "workspace missing or too small";
    case MILO_ERR_ARG: return "an enum or flag argument has no meaning";
    case MILO_ERR_HIP: return "a HIP runtime call or launch failed";
    default: return "unknown status";
  }
}

const char* milo_last_error(void) { return g_err; }

int64_t milo_packed_words(int64_t rows, int64_t K) { return 3 * rows * K / 32; }
int64_t milo_sz_words(int64_t rows, int64_t K) { return rows * K / 64; }

int32_t milo_quantize_rtn_int3_grouped(const float* W, int64_t rows, int64_t K, int32_t group,
                                       uint8_t* codes, uint16_t* scale, uint16_t* zero, void* stream) {
  g_err[0] = 0;
  if (!W || !codes || !scale || !zero) MILO_FAIL(MILO_ERR_NULL, "W, codes, scale, zero are required");
  if (group < 1 || group > 64) MILO_FAIL(MILO_ERR_SHAPE, "group=%d outside 1..64", group);
  if (rows < 1 || K < group || K % group || rows > (1ll << 31) || K > (1ll << 31))
    MILO_FAIL(MILO_ERR_SHAPE, "rows=%lld K=%lld: need rows >= 1, K >= group, K %% group == 0 (group %d)",
              (long long)rows, (long long)K, group);
  if (!aligned(W, 4) || !aligned(scale, 2) || !aligned(zero, 2))
    MILO_FAIL(MILO_ERR_ALIGN, "W must be 4-byte and scale/zero 2-byte aligned");
  return launch_quantize(W, rows, K, group, codes, scale, zero, (hipStream_t)stream);
}

int32_t milo_quantize_rtn_int3(const float* W, int64_t rows, int64_t K, uint8_t* codes,
                               uint16_t* scale, uint16_t* zero, void* stream) {
  return milo_quantize_rtn_int3_grouped(W, rows, K, kGroup, codes, scale, zero, stream);
}

int32_t milo_quantize_hqq_int3(const float* W, int64_t rows, int64_t K, int32_t iters, double p_norm,
                               double beta, double kappa, uint8_t* codes, uint16_t* scale, uint16_t* zero,
                               void* stream) {
  g_err[0] = 0;
  if (!W || !codes || !scale || !zero) MILO_FAIL(MILO_ERR_NULL, "W, codes, scale, zero are required");
  if (rows < 1 || K < 64 || K % 64 || rows > (1ll << 31) || K > (1ll << 31))
    MILO_FAIL(MILO_ERR_SHAPE, "rows=%lld K=%lld: need rows >= 1, K >= 64, K %% 64 == 0", (long long)rows,
              (long long)K);
  if (iters < 0 || iters > 1000 || !(p_norm > 0.0 && p_norm <= 1.0) || !(beta > 0.0) || !(kappa >= 1.0))
    MILO_FAIL(MILO_ERR_ARG, "iters=%d p=%g beta=%g kappa=%g: need 0 <= iters <= 1000, 0 < p <= 1, beta > 0, "
              "kappa >= 1", iters, p_norm, beta, kappa);
  if (!aligned(W, 16) || !aligned(codes, 8) || !aligned(scale, 2) || !aligned(zero, 2))
    MILO_FAIL(MILO_ERR_ALIGN, "W must be 16-byte, codes 8-byte and scale/zero 2-byte aligned");
  return launch_hqq(W, rows, K, iters, p_norm, beta, kappa, codes, scale, zero, (hipStream_t)stream);
}

int64_t milo_lr_v_words(int32_t max_rank, int64_t K) { return 3 * (int64_t)max_rank * K / 32; }
int64_t milo_lr_v_sz_words(int32_t max_rank, int64_t K) { return (int64_t)max_rank * K / 64; }
int64_t milo_lr_u_words(int64_t N, int32_t max_rank) { return 3 * N * (int64_t)round_up(max_rank, 32) / 32; }
int64_t milo_lr_u_sz_words(int64_t N) { return N; }

int32_t milo_pack_lr_int3(const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                          const uint8_t* u_codes, const uint16_t* u_scale, const uint16_t* u_zero,
                          int64_t N, int64_t K, int32_t rank, int32_t max_rank, uint32_t* vq,
                          uint32_t* vsz, uint32_t* uq, uint32_t* usz, void* stream) {
  g_err[0] = 0;
  if (!vq || !vsz || !uq || !usz) MILO_FAIL(MILO_ERR_NULL, "vq, vsz, uq, usz are required");
  if (rank > 0 && (!v_codes || !v_scale || !v_zero || !u_codes || !u_scale || !u_zero))
    MILO_FAIL(MILO_ERR_NULL, "codes, scales and zeros of both factors are required when rank > 0");
  if (N <= 0 || K <= 0 || N % 64 || K % 128 || N > 65536 || K > 65536)
    MILO_FAIL(MILO_ERR_SHAPE, "N=%lld K=%lld: need N %% 64 == 0, K %% 128 == 0, both in 1..65536",
              (long long)N, (long long)K);
  if (max_rank < 8 || max_rank > kMaxRank || max_rank % 8 || rank < 0 || rank > max_rank || rank % 8)
    MILO_FAIL(MILO_ERR_RANK, "rank=%d max_rank=%d: need 0 <= rank <= max_rank, 8 <= max_rank <= 64, "
              "multiples of 8", rank, max_rank);
  if (!aligned(vq, 16) || !aligned(vsz, 16) || !aligned(uq, 16) || !aligned(usz, 16))
    MILO_FAIL(MILO_ERR_ALIGN, "vq, vsz, uq, usz must be 16-byte aligned");
  if (!aligned(v_scale, 2) || !aligned(v_zero, 2) || !aligned(u_scale, 2) || !aligned(u_zero, 2))
    MILO_FAIL(MILO_ERR_ALIGN, "scales and zeros must be 2-byte aligned");
  return launch_pack_lr(v_codes, v_scale, v_zero, u_codes, u_scale, u_zero, N, K, rank, max_rank, vq,
                        vsz, uq, usz, (hipStream_t)stream);
}

int32_t milo_pack_int3(const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                       int64_t rows, int64_t K, uint32_t* packed, uint32_t* sz, void* stream) {
  g_err[0] = 0;
  if (!codes || !scale || !zero || !packed || !sz)
    MILO_FAIL(MILO_ERR_NULL, "codes, scale, zero, packed, sz are required");
  if (rows <= 0 || K <= 0 || rows % 64 || K % 128 || rows > (1ll << 31) || K > (1ll << 31))
    MILO_FAIL(MILO_ERR_SHAPE, "rows=%lld K=%lld: need rows %% 64 == 0 and K %% 128 == 0",
              (long long)rows, (long long)K);
  if (!aligned(codes, 16) || !aligned(packed, 16) || !aligned(sz, 16) || !aligned(scale, 2) || !aligned(zero, 2))
    MILO_FAIL(MILO_ERR_ALIGN, "codes, packed, sz must be 16-byte aligned");
  return launch_pack(codes, scale, zero, rows, K, packed, sz, (hipStream_t)stream);
}

static int32_t check_lowrank_shape(int64_t N, int64_t K, int32_t rank, int32_t oversample) {
  if (N < 1 || K < 1 || N > (1 << 20) || K > (1 << 20))
    MILO_FAIL(MILO_ERR_SHAPE, "N=%lld K=%lld outside 1..1048576", (long long)N, (long long)K);
  if (rank < 0 || rank > kMaxRank) MILO_FAIL(MILO_ERR_RANK, "rank=%d outside 0..64", rank);
  if (oversample < 0 || rank + oversample > 80)
    MILO_FAIL(MILO_ERR_RANK, "rank + oversample = %d outside rank..80", rank + oversample);
  if (rank > 0 && (rank + oversample > N || rank + oversample > K))
    MILO_FAIL(MILO_ERR_SHAPE, "rank + oversample = %d exceeds min(N, K)", rank + oversample);
  return MILO_OK;
}

size_t milo_lowrank_svd_workspace_bytes(int64_t N, int64_t K, int32_t rank, int32_t oversample) {
  if (check_lowrank_shape(N, K, rank, oversample) != MILO_OK || rank == 0) return 0;
  return svd_workspace_bytes(N, K, rank + oversample);
}

int32_t milo_lowrank_svd(const float* R, int64_t N, int64_t K, int32_t rank, int32_t oversample,
                         int32_t power_iters, const float* omega, float* U, float* V, float* sigma,
                         void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int32_t rc = check_lowrank_shape(N, K, rank, oversample);
  if (rc != MILO_OK) return rc;
  if (power_iters < 0 || power_iters > 8) MILO_FAIL(MILO_ERR_ARG, "power_iters=%d outside 0..8", power_iters);
  if (rank == 0) return MILO_OK;
  if (!R || !omega || !U || !V || !sigma) MILO_FAIL(MILO_ERR_NULL, "R, omega, U, V, sigma are required");
  if (!aligned(R, 4) || !aligned(omega, 4) || !aligned(U, 4) || !aligned(V, 4) || !aligned(sigma, 4))
    MILO_FAIL(MILO_ERR_ALIGN, "float arrays must be 4-byte aligned");
  const size_t need = svd_workspace_bytes(N, K, rank + oversample);
  if (!workspace || ws_bytes < need) MILO_FAIL(MILO_ERR_WORKSPACE, "svd workspace %zu bytes < required %zu", ws_bytes, need);
  if (!aligned(workspace, 256)) MILO_FAIL(MILO_ERR_ALIGN, "workspace must be 256-byte aligned");
  return run_lowrank_svd(R, N, K, rank, rank + oversample, power_iters, omega, U, V, sigma, (char*)workspace,
                         (hipStream_t)stream);
}

size_t milo_build_compensator_workspace_bytes(int64_t N, int64_t K, int32_t rank, int32_t oversample) {
  if (check_lowrank_shape(N, K, rank, oversample) != MILO_OK) return 0;
  return build_workspace_bytes(N, K, rank + oversample);
}

int32_t milo_build_compensator(const float* W, int64_t N, int64_t K, int32_t rank, int32_t iters,
                               int32_t oversample, int32_t power_iters, int32_t quantizer,
                               const float* omega, uint8_t* codes,
                               uint16_t* scale, uint16_t* zero, float* U, float* V, float* sigma,
                               void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int32_t rc = check_lowrank_shape(N, K, rank, oversample);
  if (rc != MILO_OK) return rc;
  if (K % kGroup) MILO_FAIL(MILO_ERR_SHAPE, "K=%lld must be a multiple of 64", (long long)K);
  if (iters < 1 || iters > 16) MILO_FAIL(MILO_ERR_ARG, "iters=%d outside 1..16", iters);
  if (power_iters < 0 || power_iters > 8) MILO_FAIL(MILO_ERR_ARG, "power_iters=%d outside 0..8", power_iters);
  if (quantizer != MILO_QUANT_RTN && quantizer != MILO_QUANT_HQQ)
    MILO_FAIL(MILO_ERR_ARG, "unknown quantizer %d", quantizer);
  if (!W || !codes || !scale || !zero) MILO_FAIL(MILO_ERR_NULL, "W, codes, scale, zero are required");
  if (rank > 0 && (!omega || !U || !V || !sigma))
    MILO_FAIL(MILO_ERR_NULL, "omega, U, V, sigma are required when rank > 0");
  if (!aligned(W, 4) || !aligned(scale, 2) || !aligned(zero, 2) || !aligned(omega, 4) || !aligned(U, 4) ||
      !aligned(V, 4) || !aligned(sigma, 4))
    MILO_FAIL(MILO_ERR_ALIGN, "W, omega, U, V, sigma 4-byte and scale, zero 2-byte aligned");
  const size_t need = build_workspace_bytes(N, K, rank + oversample);
  if (!workspace || ws_bytes < need)
    MILO_FAIL(MILO_ERR_WORKSPACE, "build workspace %zu bytes < required %zu", ws_bytes, need);
  if (!aligned(workspace, 256)) MILO_FAIL(MILO_ERR_ALIGN, "workspace must be 256-byte aligned");
  return run_build(W, N, K, rank, iters, rank + oversample, power_iters, omega, quantizer, codes, scale, zero, U,
                   V, sigma,
                   (char*)workspace, (hipStream_t)stream);
}

size_t milo_weight_kurtosis_workspace_bytes(int64_t count) {
  return count >= 1 && count <= 65535 ? kurtosis_workspace_bytes(count) : 0;
}

int32_t milo_weight_kurtosis(const float* W, int64_t count, int64_t elems, double* kurtosis, double* mean,
                             void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!W || !kurtosis) MILO_FAIL(MILO_ERR_NULL, "W and kurtosis are required");
  if (count < 1 || count > 65535 || elems < 4 || elems % 4 || elems > (1ll << 40))
    MILO_FAIL(MILO_ERR_SHAPE, "count=%lld elems=%lld: need 1 <= count <= 65535, elems >= 4, elems %% 4 == 0",
              (long long)count, (long long)elems);
  if (!aligned(W, 16) || !aligned(kurtosis, 8) || !aligned(mean, 8))
    MILO_FAIL(MILO_ERR_ALIGN, "W must be 16-byte and kurtosis/mean 8-byte aligned");
  const size_t need = kurtosis_workspace_bytes(count);
  if (!workspace || ws_bytes < need)
    MILO_FAIL(MILO_ERR_WORKSPACE, "kurtosis workspace %zu bytes < required %zu", ws_bytes, need);
  if (!aligned(workspace, 8)) MILO_FAIL(MILO_ERR_ALIGN, "workspace must be 8-byte aligned");
  return launch_kurtosis(W, count, elems, kurtosis, mean, (char*)workspace, (hipStream_t)stream);
}

int32_t milo_expert_counts(const int32_t* offsets, int32_t num_experts, int64_t* counts, void* stream) {
  g_err[0] = 0;
  if (!offsets || !counts) MILO_FAIL(MILO_ERR_NULL, "offsets and counts are required");
  if (num_experts < 1 || num_experts > 256) MILO_FAIL(MILO_ERR_SHAPE, "num_experts=%d outside 1..256", num_experts);
  if (!aligned(offsets, 4) || !aligned(counts, 8)) MILO_FAIL(MILO_ERR_ALIGN, "offsets 4-, counts 8-byte aligned");
  return launch_expert_counts(offsets, num_experts, counts, (hipStream_t)stream);
}

int32_t milo_rank_policy(const double* kurtosis, const double* frequency, const int32_t* dense, int32_t n,
                         int32_t total_rank, int32_t r_min, int32_t r_max, int32_t step, int32_t* ranks) {
  g_err[0] = 0;
  if (n < 0) MILO_FAIL(MILO_ERR_SHAPE, "n=%d < 0", n);
  if (n == 0) return MILO_OK;
  if (!kurtosis || !frequency || !dense || !ranks) MILO_FAIL(MILO_ERR_NULL, "all arrays are required");
  if (step < 1 || r_min < 0 || r_min > r_max || r_max > kMaxRank || r_min % step || r_max % step ||
      total_rank < 0 || total_rank % step)
    MILO_FAIL(MILO_ERR_RANK, "step=%d r_min=%d r_max=%d total_rank=%d: need multiples of step, "
              "0 <= r_min <= r_max <= 64", step, r_min, r_max, total_rank);
  rank_policy_host(kurtosis, frequency, dense, n, total_rank, r_min, r_max, step, ranks);
  return MILO_OK;
}

size_t milo_route_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t S) {
  (void)k;
  if (T <= 256) return 0;
  const size_t nb = ((size_t)T + 255) / 256;
  return round_up(nb * (size_t)(E + S) * 4, 256);
}

int32_t milo_route_sort(const float* logits, int32_t T, int32_t E, int32_t k, int32_t S,
                        int32_t renormalize, int32_t* topk_ids, float* topk_w, float* slot_w,
                        int32_t* sorted_pairs, int32_t* pair_pos, int32_t* offsets,
                        void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!logits || !topk_ids || !topk_w || !slot_w || !sorted_pairs || !pair_pos || !offsets)
    MILO_FAIL(MILO_ERR_NULL, "logits and all outputs are required");
  if (T < 1 || T > 65536) MILO_FAIL(MILO_ERR_SHAPE, "T=%d outside 1..65536", T);
  if (E < 1 || k < 1 || k > E || k > 8 || S < 0 || E + S > 256 || k + S > 16)
    MILO_FAIL(MILO_ERR_SHAPE, "E=%d k=%d S=%d: need 1 <= k <= min(E, 8), E + S <= 256, k + S <= 16", E, k, S);
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(slot_w, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(pair_pos, 4) || !aligned(offsets, 4))
    MILO_FAIL(MILO_ERR_ALIGN, "routing arrays must be 4-byte aligned");
  const size_t need = milo_route_workspace_bytes(T, E, k, S);
  if (need && (!workspace || ws_bytes < need))
    MILO_FAIL(MILO_ERR_WORKSPACE, "route workspace %zu bytes < required %zu", ws_bytes, need);
  if (need && !aligned(workspace, 4)) MILO_FAIL(MILO_ERR_ALIGN, "workspace must be 4-byte aligned");
  return launch_route(logits, T, E, k, S, renormalize ? 1 : 0, topk_ids, topk_w, slot_w, sorted_pairs,
                      pair_pos, offsets, workspace, (hipStream_t)stream);
}

size_t milo_moe_gemm_workspace_bytes(const milo_gemm_desc* d) {
  if (validate_gemm(d) != MILO_OK) return 0;
  GemmPlan p;
  if (plan_gemm(d, &p) != MILO_OK) return 0;
  return p.total;
}

static int32_t prepare_call(const milo_gemm_desc* d, void* workspace, size_t ws_bytes, GemmPlan* p) {
  int32_t rc = validate_gemm(d);
  if (rc != MILO_OK) return rc;
  if (d->flags & ~MILO_GEMM_PREPASS_DONE) MILO_FAIL(MILO_ERR_ARG, "unknown flags 0x%x", d->flags);
  rc = plan_gemm(d, p);
  if (rc != MILO_OK) return rc;
  if (d->num_pairs == 0) return MILO_OK;
  if (p->total && (!workspace || ws_bytes < p->total))
    MILO_FAIL(MILO_ERR_WORKSPACE, "gemm workspace %zu bytes < required %zu", ws_bytes, p->total);
  if (p->total && !aligned(workspace, 256)) MILO_FAIL(MILO_ERR_ALIGN, "workspace must be 256-byte aligned");
  return MILO_OK;
}

int32_t milo_moe_lowrank_prepass(const milo_gemm_desc* d, void* workspace, size_t ws_bytes,
                                 void* stream) {
  g_err[0] = 0;
  GemmPlan p;
  int32_t rc = prepare_call(d, workspace, ws_bytes, &p);
  if (rc != MILO_OK || d->num_pairs == 0) return rc;
  return launch_lowrank(d, p, (char*)workspace, (hipStream_t)stream);
}

int32_t milo_moe_w3a16_lowrank_gemm(const milo_gemm_desc* d, void* workspace, size_t ws_bytes,
                                    void* stream) {
  g_err[0] = 0;
  GemmPlan p;
  int32_t rc = prepare_call(d, workspace, ws_bytes, &p);
  if (rc != MILO_OK || d->num_pairs == 0) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (!(d->flags & MILO_GEMM_PREPASS_DONE)) {
    rc = launch_lowrank(d, p, ws, st);
    if (rc != MILO_OK) return rc;
  }
  rc = launch_gemm_decode(d, p, ws, st);
  if (rc != MILO_OK) return rc;
  return launch_gemm_prefill(d, p, ws, st);
}

}  // extern "C"

namespace milo {

// Library-owned scratch of milo_moe_w3a16_lowrank_gemm_static.  Host code
// never uses the array's name as an address: each device's copy is looked
// up once (hipGetSymbolAddress, with that device current) and the pointer
// kept per device.
static __device__ __align__(256) unsigned char scratch[MILO_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices] = {nullptr};
static std::mutex g_scratch_mu;

static int32_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) MILO_FAIL(MILO_ERR_HIP, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) MILO_FAIL(MILO_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL on device %d", dev);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MILO_OK;
}

}  // namespace milo

extern "C" {

int32_t milo_moe_w3a16_lowrank_gemm_static(const milo_gemm_desc* d, void* stream) {
  g_err[0] = 0;
  int32_t rc = validate_gemm(d);
  if (rc != MILO_OK) return rc;
  if (d->flags) MILO_FAIL(MILO_ERR_ARG, "flags=0x%x: the static-workspace call runs the whole GEMM (flags must be 0)",
                          d->flags);
  GemmPlan p;
  rc = plan_gemm(d, &p);
  if (rc != MILO_OK || d->num_pairs == 0) return rc;
  if (p.total > MILO_STATIC_WORKSPACE_BYTES)
    MILO_FAIL(MILO_ERR_WORKSPACE, "this GEMM needs %zu bytes of workspace, more than the library's static %zu; "
              "use milo_moe_w3a16_lowrank_gemm with a caller workspace", p.total,
              (size_t)MILO_STATIC_WORKSPACE_BYTES);
  void* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc != MILO_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  rc = launch_lowrank(d, p, (char*)ws, st);
  if (rc != MILO_OK) return rc;
  rc = launch_gemm_decode(d, p, (char*)ws, st);
  if (rc != MILO_OK) return rc;
  return launch_gemm_prefill(d, p, (char*)ws, st);
}

int32_t milo_moe_combine(const float* y, int32_t T, int32_t slots, int32_t H, uint16_t* out,
                         void* stream) {
  g_err[0] = 0;
  if (!y || !out) MILO_FAIL(MILO_ERR_NULL, "y and out are required");
  if (T < 1 || slots < 1 || slots > 16 || H < 4 || H % 4)
    MILO_FAIL(MILO_ERR_SHAPE, "T=%d slots=%d H=%d: need T >= 1, 1 <= slots <= 16, H %% 4 == 0", T, slots, H);
  if (!aligned(y, 16) || !aligned(out, 16)) MILO_FAIL(MILO_ERR_ALIGN, "y and out must be 16-byte aligned");
  return launch_combine(y, T, slots, H, out, (hipStream_t)stream);
}

}  // extern "C"
