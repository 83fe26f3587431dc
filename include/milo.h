/*
 * milo.h -- C ABI of libmilo, an MI355X (gfx950) implementation of the MiLo
 * W3A16 + low-rank-compensated MoE expert GEMM.
 *
 * Sources ("the pages"):
 *   [talk] "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
 *          Compensators", write-up of the MLSys 2025 talk: sections Background,
 *          Technical Deep Dive (MiLo Algorithm, MiLo Kernel), Experimental
 *          Setup & Results.
 *   [abs]  the arXiv abstract of the same paper (2504.02658).
 *
 * General rules for every entry point:
 *   - All tensor pointers are DEVICE pointers to caller-owned memory (the
 *     library never allocates or frees).  Scalars and descriptor structs are
 *     host values.  `stream` is a hipStream_t (NULL = default stream).
 *   - Calls are asynchronous: they enqueue kernels on `stream` and return.
 *     No entry point synchronises the host with the device.
 *   - Every shape, pointer, alignment and workspace check runs on the host
 *     before anything is enqueued; on an error nothing is enqueued and the
 *     return value is a nonzero milo_status.  Launch failures return
 *     MILO_ERR_HIP.  Details of the last error of the calling thread are in
 *     milo_last_error().  Device faults surface at the caller's next
 *     synchronisation, as with any HIP kernel.
 *   - float16 values are passed as uint16_t bit patterns (IEEE binary16).
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics; fixed reduction orders).
 */
#ifndef MILO_H
#define MILO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MILO_ABI_VERSION 2
#define MILO_LAYOUT_VERSION 1

typedef enum milo_status {
  MILO_OK = 0,
  MILO_ERR_NULL = 1,       /* a required pointer is NULL                   */
  MILO_ERR_SHAPE = 2,      /* a size violates the documented constraints   */
  MILO_ERR_ALIGN = 3,      /* a pointer is not aligned as documented       */
  MILO_ERR_RANK = 4,       /* compensator rank outside the supported range */
  MILO_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required   */
  MILO_ERR_ARG = 6,        /* an enum or flag argument has no meaning      */
  MILO_ERR_HIP = 7         /* a HIP runtime call or launch failed          */
} milo_status;

int32_t milo_abi_version(void);      /* MILO_ABI_VERSION    */
int32_t milo_layout_version(void);   /* MILO_LAYOUT_VERSION */
/* Static description of a status code (never NULL). */
const char* milo_status_string(int32_t status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* milo_last_error(void);

/* ======================================================================
 * Offline weight preparation (not on the timed path)
 * ====================================================================== */

/*
 * Group-wise asymmetric int3 round-to-nearest quantization.
 * [talk] Background names RTN as the simplest calibration-free quantizer;
 * MiLo Algorithm / Key Findings describe int3 weights with an asymmetric
 * zero point.  Per row and group of 64 consecutive columns, in float64:
 *     lo, hi = min, max;   s = f16_rne((hi - lo) / 7), s = 1 if that is 0;
 *     z = f16_rne(clamp(-lo / s, -65504, 65504));
 *     q = clamp(rint(w / s + z), 0, 7)    (round half to even)
 * and the weight is represented as (q - z) * s.
 *
 * W      : float32 [rows][K], row-major.
 * codes  : out, uint8 [rows][K] (values 0..7).
 * scale  : out, float16 bits [rows][K/64].
 * zero   : out, float16 bits [rows][K/64].
 * Constraints: rows >= 1, K >= 64, K % 64 == 0.  W must be finite.
 */
int32_t milo_quantize_rtn_int3(const float* W, int64_t rows, int64_t K,
                               uint8_t* codes, uint16_t* scale, uint16_t* zero,
                               void* stream);

/*
 * The same quantizer with groups of `group` consecutive columns (1 <= group
 * <= 64, K % group == 0); scale and zero are [rows][K/group].  With
 * group == 64 it is milo_quantize_rtn_int3.  Used for the int3 compensator
 * factors (see milo_pack_lr_int3): V rows in groups of 64, U rows in one
 * group of the expert's rank.
 */
int32_t milo_quantize_rtn_int3_grouped(const float* W, int64_t rows, int64_t K,
                                       int32_t group, uint8_t* codes,
                                       uint16_t* scale, uint16_t* zero,
                                       void* stream);

/*
 * HQQ-style int3 quantization ([talk] Key Findings / MiLo Algorithm: MiLo's
 * initial, calibration-free quantizer is HQQ; the method is Badri & Shaji,
 * "Half-Quadratic Quantization of Large Machine Learning Models", 2023):
 * per row and group of 64 columns, the RTN scale of milo_quantize_rtn_int3
 * is kept and the zero point is optimized for a sparsity-promoting l_p error
 * by half-quadratic splitting, in float64:
 *     z_0 = RTN zero point;  repeat iters times:
 *         q = clamp(rint(w / s + z), 0, 7);  x = w - (q - z) s
 *         W_e = sign(x) max(|x| - |x|^(p_norm - 1) / beta, 0)
 *         z = mean over the group of (q - (w - W_e) / s);  beta *= kappa
 *     after each iteration the fp16 value of z is a candidate, scored by the
 *     group's mean absolute error with codes chosen at it; the best
 *     candidate (RTN's zero point first) is stored, with its codes.
 * So no group's mean absolute error exceeds RTN's.  Published defaults:
 * p_norm 0.7, beta 10, kappa 1.01, 20 iterations; iters 0 reproduces RTN.
 * Arguments and outputs as milo_quantize_rtn_int3, except alignment: W must
 * be 16-byte and codes 8-byte aligned (MILO_ERR_ALIGN otherwise).
 */
int32_t milo_quantize_hqq_int3(const float* W, int64_t rows, int64_t K,
                               int32_t iters, double p_norm, double beta,
                               double kappa, uint8_t* codes, uint16_t* scale,
                               uint16_t* zero, void* stream);

/* Number of uint32 words of the packed codes of a rows x K matrix: 3*rows*K/32. */
int64_t milo_packed_words(int64_t rows, int64_t K);
/* Number of uint32 words of the tiled scale/zero of a rows x K matrix: rows*K/64. */
int64_t milo_sz_words(int64_t rows, int64_t K);

/*
 * Repack int3 codes into packed layout v1 and tile the scale/zero pairs.
 * [talk] MiLo Kernel, "Bit Packing": 32 three-bit values are stored in three
 * 32-bit words without wasting a bit.  Layout v1 keeps that density with its
 * own bit assignment:
 *   Tile (rt, kb) = rows [64 rt, 64 rt + 64) x columns [128 kb, 128 kb + 128),
 *   tile index t = rt * (K/128) + kb, 768 words at packed[768 t ...].
 *   Word 256 p + 4 L + i of a tile (plane p = 0..2, lane L = 0..63, row group
 *   i = 0..3) is word p of the triplet holding row 64 rt + 16 i + (L mod 16),
 *   codes c = 0..31 at column 128 kb + 32 (c div 8) + 8 (L div 16) + (c mod 8).
 *   Code c = 2 pi + h (pair pi, half h): for pi < 15 it occupies bits
 *   [16 h + 1 + 3 (pi mod 5), +3) of word pi div 5; for pi = 15 bit b of the
 *   code is bit 16 h of word b.
 *   Scale/zero: sz[128 t + 8 (r mod 16) + 2 ((r mod 64) div 16) + (g mod 2)] =
 *   scale_bits | zero_bits << 16 for row r, group g (t from r and g div 2).
 * A batch of experts with equal shapes is packed in one call by stacking
 * them as rows (expert e's rows start at e*N; N % 64 == 0 keeps tiles inside
 * one expert), giving expert e's packed words at e * milo_packed_words(N, K).
 *
 * codes  : uint8 [rows][K], only the low 3 bits are used.
 * scale, zero : float16 bits [rows][K/64].
 * packed : out, uint32 [milo_packed_words(rows, K)], 16-byte aligned.
 * sz     : out, uint32 [milo_sz_words(rows, K)], 16-byte aligned.
 * Constraints: rows % 64 == 0, K % 128 == 0, rows, K > 0.
 */
int32_t milo_pack_int3(const uint8_t* codes, const uint16_t* scale,
                       const uint16_t* zero, int64_t rows, int64_t K,
                       uint32_t* packed, uint32_t* sz, void* stream);

/*
 * int3 compensator factors of one expert.
 * [talk] MiLo Algorithm, last step, and Experimental Setup & Results,
 * "Compensator Quantization": the low-rank factors U (out x R) and V (R x in)
 * are themselves quantized to int3 by simple asymmetric linear quantization.
 * Quantizer: milo_quantize_rtn_int3_grouped, with the groups along the
 * dimension each factor is summed over: V rows (one per rank j) in groups of
 * 64 along K; U rows (one per output n) in one group of the expert's r ranks.
 * Triplets keep the layout v1 bit assignment (32 codes in 3 words; code
 * c = 2 pi + h at bits [16 h + 1 + 3 (pi mod 5), +3) of word pi div 5 for
 * pi < 15, bit b of codes 30 + h at bit 16 h of word b).
 *
 * V layout: max_rank rows (rank rows j), each its K/32 triplets in order
 *   tau = 4 kb + kq (kb = column block of 128, kq = 0..3); triplet tau of
 *   row j is at vq[3 (j K/32 + tau) ...], its code c at column
 *   128 kb + 32 (c div 8) + 8 kq + (c mod 8).  Scale/zero:
 *   vsz[j (K/64) + gg] = scale | zero << 16 for row j, group gg.  Rows
 *   j >= rank: codes 0, scale 1, zero 0.  milo_lr_v_words /
 *   milo_lr_v_sz_words words per expert.
 * U layout: ranks padded to R32 = max_rank rounded up to 32.  Tile (nt, jt) =
 *   rows [64 nt, +64) x ranks [32 jt, +32), index t = nt (R32/32) + jt, 192
 *   words.  Word 64 p + L is word p of the triplet whose code c is U[n][j],
 *   n = 64 nt + 16 (c div 8) + (L mod 16), j = 32 jt + 8 (L div 16) + (c mod 8)
 *   (one lane's triplet is exactly its matrix-core B operand of 4 x 8 values).
 *   Ranks j >= rank: code 0.  Scale/zero, one per row:
 *   usz[64 (n div 64) + 4 (n mod 16) + (n mod 64) div 16].
 *   milo_lr_u_words / milo_lr_u_sz_words (= N) words per expert.
 */
int64_t milo_lr_v_words(int32_t max_rank, int64_t K);
int64_t milo_lr_v_sz_words(int32_t max_rank, int64_t K);
int64_t milo_lr_u_words(int64_t N, int32_t max_rank);
int64_t milo_lr_u_sz_words(int64_t N);

/*
 * Pack one expert's quantized compensator factors into the layouts above.
 * v_codes : uint8 [rank][K];  v_scale, v_zero : fp16 bits [rank][K/64].
 * u_codes : uint8 [N][rank];  u_scale, u_zero : fp16 bits [N] (one group).
 * vq, vsz, uq, usz : out, milo_lr_*_words(...) uint32 each, 16-byte aligned.
 * Every output word is written (padding included).  The v_* / u_* inputs
 * may be NULL when rank == 0.
 * Constraints: N % 64 == 0, K % 128 == 0, 0 <= rank <= max_rank <= 64, both
 * multiples of 8, max_rank >= 8.
 */
int32_t milo_pack_lr_int3(const uint8_t* v_codes, const uint16_t* v_scale,
                          const uint16_t* v_zero, const uint8_t* u_codes,
                          const uint16_t* u_scale, const uint16_t* u_zero,
                          int64_t N, int64_t K, int32_t rank, int32_t max_rank,
                          uint32_t* vq, uint32_t* vsz, uint32_t* uq,
                          uint32_t* usz, void* stream);

/* ======================================================================
 * Offline compensator construction
 * ====================================================================== */

/*
 * Rank-r approximation of a residual matrix, R ~ U V, by randomized subspace
 * iteration (Halko, Martinsson & Tropp, "Finding structure with randomness",
 * SIAM Review 2011, Algorithm 4.4) -- the "SVD of the residual" step of
 * [talk] MiLo Algorithm, Compensation Generation, which keeps the top-R
 * singular values and vectors.  With l = rank + oversample:
 *     Y = R Omega;  Q = orth(Y);  power_iters times: Z = orth(R^T Q), Q = orth(R Z)
 *     B = Q^T R;  B B^T = W diag(lambda) W^T (eigenvalues descending)
 *     sigma = lambda^(1/2) of the top rank;  U = Q W_r diag(sigma^(1/2));
 *     V = diag(sigma^(-1/2)) W_r^T B
 * orth() is CholeskyQR2; fp32 data, fp64 for the l x l factorizations.
 * U V is the rank-r approximation; the split is balanced (column norms of U =
 * row norms of V = sigma^(1/2)); directions with sigma = 0 give zero factors.
 *
 * R     : float32 [N][K].
 * omega : float32 [l][K], the Gaussian test matrix, transposed (the caller
 *         draws it, e.g. N(0, 1)).
 * U     : out, float32 [N][rank];  V : out, float32 [rank][K];
 * sigma : out, float32 [rank], descending.
 * workspace : milo_lowrank_svd_workspace_bytes(...) bytes, 256-byte aligned.
 * Constraints: 0 <= rank <= 64, oversample >= 0, rank + oversample <= 80 and
 *   <= min(N, K), N, K <= 2^20, 0 <= power_iters <= 8.  rank == 0 is a no-op.
 */
size_t milo_lowrank_svd_workspace_bytes(int64_t N, int64_t K, int32_t rank,
                                        int32_t oversample);
int32_t milo_lowrank_svd(const float* R, int64_t N, int64_t K, int32_t rank,
                         int32_t oversample, int32_t power_iters,
                         const float* omega, float* U, float* V, float* sigma,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Quantize-and-compensate refinement of one weight matrix, [talk] MiLo
 * Algorithm (Compensation Generation; the iterative optimization that
 * recomputes W_quant from U V and U V from the new residual):
 *     L_0 = 0;  for t = 1..iters:
 *         (codes, scale, zero) = quantize(W - L_{t-1}), quantize =
 *             milo_quantize_rtn_int3 (quantizer MILO_QUANT_RTN) or
 *             milo_quantize_hqq_int3 with its published defaults
 *             (MILO_QUANT_HQQ, the pages' initial quantizer)
 *         R_t = W - (codes - zero) scale
 *         (U, V, sigma) = milo_lowrank_svd(R_t, test matrix omega[t-1]);  L_t = U V
 * and returns the last quantization and factors: W ~ deq(codes) + U V, i.e.
 * the compensator of milo_weights with U [N][rank] and V [rank][K].
 *
 * W     : float32 [N][K].
 * omega : float32 [iters][l][K] test matrices (NULL when rank == 0).
 * codes : out, uint8 [N][K];  scale, zero : out, fp16 bits [N][K/64].
 * U, V, sigma : out as in milo_lowrank_svd (unused when rank == 0).
 * workspace : milo_build_compensator_workspace_bytes(...) bytes (holds one
 *   N x K float32 residual), 256-byte aligned.
 * Constraints: those of milo_lowrank_svd, K % 64 == 0, 1 <= iters <= 16.
 */
enum { MILO_QUANT_RTN = 0, MILO_QUANT_HQQ = 1 };
size_t milo_build_compensator_workspace_bytes(int64_t N, int64_t K, int32_t rank,
                                              int32_t oversample);
int32_t milo_build_compensator(const float* W, int64_t N, int64_t K, int32_t rank,
                               int32_t iters, int32_t oversample,
                               int32_t power_iters, int32_t quantizer,
                               const float* omega,
                               uint8_t* codes, uint16_t* scale, uint16_t* zero,
                               float* U, float* V, float* sigma, void* workspace,
                               size_t ws_bytes, void* stream);

/*
 * Adaptive compensator ranks, [talk] MiLo Algorithm, "Mixture of Low-Rank
 * Compensators and Adaptive Rank Selection": dense (always-activated) parts,
 * frequently activated experts and weights with a higher kurtosis get higher
 * ranks.  The pages give no formula; the policy implemented is
 *     score_m = (dense_m ? 1 : frequency_m) * kurtosis_m / 3
 * and a budget of total_rank rank units is apportioned in proportion to the
 * scores in steps of `step`, each rank clipped to [r_min, r_max], by the
 * largest-remainder method (units handed out, or taken back when r_min
 * forces it, one at a time by remainder, ties to the lower index; the score
 * sum runs left to right).
 */

/* Population kurtosis E[(w - mu)^4] / E[(w - mu)^2]^2 of each of `count`
   matrices of `elems` float32 values stored back to back (W: device,
   16-byte aligned; elems % 4 == 0).  Two streaming passes, float64
   accumulation, deterministic.  kurtosis: out, device double [count] (0 for
   a constant matrix); mean: optional out, device double [count].
   workspace: milo_weight_kurtosis_workspace_bytes(count) bytes, device. */
size_t milo_weight_kurtosis_workspace_bytes(int64_t count);
int32_t milo_weight_kurtosis(const float* W, int64_t count, int64_t elems,
                             double* kurtosis, double* mean, void* workspace,
                             size_t ws_bytes, void* stream);

/* counts[e] += offsets[e + 1] - offsets[e] for e < num_experts (device
   arrays; counts int64, caller-initialised): routed pairs per expert,
   accumulated over routing calls -- the activation frequency is counts /
   tokens. */
int32_t milo_expert_counts(const int32_t* offsets, int32_t num_experts,
                           int64_t* counts, void* stream);

/* The apportionment above on HOST arrays of n matrices (kurtosis,
   frequency: double; dense: int32 0/1) into ranks (host int32 [n]).
   Synchronous, touches no device.  Constraints: step >= 1; r_min, r_max,
   total_rank multiples of step; 0 <= r_min <= r_max <= 64.  When
   n r_min > total_rank or n r_max < total_rank the ranks sum to the nearest
   feasible total. */
int32_t milo_rank_policy(const double* kurtosis, const double* frequency,
                         const int32_t* dense, int32_t n, int32_t total_rank,
                         int32_t r_min, int32_t r_max, int32_t step,
                         int32_t* ranks);

/* ======================================================================
 * Routing
 * ====================================================================== */

/* Workspace bytes milo_route_sort needs for these sizes (may be 0). */
size_t milo_route_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t S);

/*
 * Softmax top-k routing and the expert-sorted (token, slot) pair list.
 * [talk] Background: each token activates only a subset of the experts.
 * For token t: the k largest logits (ties -> lower expert id), ordered by
 * decreasing logit; p = softmax(logits[t]) in float32; routed weight
 * w = p_j / sum over the k picks (renormalize != 0) or p_j (renormalize == 0).
 * Slot j of token t has slot index s = t*(k+S) + j; slots j >= k are the S
 * shared experts E + (j - k) with weight 1.  Pairs are sorted by
 * (expert, s).
 *
 * logits      : float32 [T][E], finite.
 * topk_ids    : out, int32 [T][k].
 * topk_w      : out, float32 [T][k].
 * slot_w      : out, float32 [T*(k+S)]   weight of each slot.
 * sorted_pairs: out, int32 [T*(k+S)]     slot indices in (expert, s) order.
 * pair_pos    : out, int32 [T*(k+S)]     inverse: pair_pos[sorted_pairs[i]] = i.
 * offsets     : out, int32 [E+S+1]       offsets[e] = #pairs with expert < e.
 * workspace   : milo_route_workspace_bytes(T,E,k,S) bytes (NULL if 0).
 * Constraints: 1 <= T <= 65536, 1 <= k <= min(E, 8), E + S <= 256,
 *              k + S <= 16.  All outputs 4-byte aligned.
 */
int32_t milo_route_sort(const float* logits, int32_t T, int32_t E, int32_t k,
                        int32_t S, int32_t renormalize, int32_t* topk_ids,
                        float* topk_w, float* slot_w, int32_t* sorted_pairs,
                        int32_t* pair_pos, int32_t* offsets, void* workspace,
                        size_t ws_bytes, void* stream);

/* ======================================================================
 * Routed W3A16 + low-rank grouped GEMM
 * ====================================================================== */

/*
 * One projection family (e.g. all experts' W1) of num_experts experts, each an
 * N x K matrix (output x input), stored as:
 *   packed : layout v1 codes, expert e at packed + e * milo_packed_words(N, K).
 *   sz     : tiled scale/zero, expert e at sz + e * milo_sz_words(N, K).
 *   U      : float16 [num_experts][N][max_rank]  the compensator factor U of
 *            [talk] MiLo Algorithm (W_out = W_quant + U V, U is out x R).
 *   V      : float16 [num_experts][max_rank][K]  the factor V (R x in).
 *   rank   : DEVICE int32 [num_experts], 0 <= rank[e] <= max_rank,
 *            rank[e] % 8 == 0.  Columns of U and rows of V at or beyond
 *            rank[e] are never read.
 *   lr_format : MILO_LR_FP16 (U, V above) or MILO_LR_INT3 (Uq, Usz, Vq, Vsz:
 *            the int3 compensator layouts of milo_pack_lr_int3, expert e at
 *            e times the per-expert word counts; U and V are then unused).
 *            Ranks at or beyond rank[e] contribute nothing whatever the
 *            padding holds.
 * The compensator pointers may be NULL when max_rank == 0.
 */
enum { MILO_LR_FP16 = 0, MILO_LR_INT3 = 1 };

typedef struct milo_weights {
  const uint32_t* packed;
  const uint32_t* sz;
  const uint16_t* U;
  const uint16_t* V;
  const int32_t* rank;
  int32_t lr_format;
  const uint32_t* Uq;
  const uint32_t* Usz;
  const uint32_t* Vq;
  const uint32_t* Vsz;
} milo_weights;

enum {
  MILO_EPI_NONE = 0,        /* y fp16 [num_pairs][N]: Y in pair order        */
  MILO_EPI_SWIGLU = 1,      /* y fp16 [num_pairs][N]: silu(Y_w0) * Y_w1      */
  MILO_EPI_ROUTE_SCALE = 2  /* y fp32 [y_rows][N]: row sorted_pairs[i] gets
                               Y_i * slot_w[sorted_pairs[i]]                */
};
enum { MILO_PATH_AUTO = 0, MILO_PATH_DECODE = 1, MILO_PATH_PREFILL = 2 };

typedef struct milo_gemm_desc {
  int32_t num_experts;          /* experts in the weight arrays (E + S)       */
  int32_t N, K;                 /* output and input features of each expert   */
  int32_t max_rank;             /* 0..64, multiple of 8                       */
  int32_t n_w;                  /* 1, or 2 for MILO_EPI_SWIGLU (w[0]=gate W1,
                                   w[1]=up W3)                                 */
  milo_weights w[2];
  const uint16_t* x;            /* fp16 [x_rows][K]                           */
  int32_t x_rows;
  int32_t gather_div;           /* >0: pair i reads x row sorted_pairs[i] /
                                   gather_div; 0: pair i reads x row i        */
  const int32_t* sorted_pairs;  /* int32 [num_pairs] (may be NULL if
                                   gather_div == 0 and epilogue != ROUTE_SCALE) */
  const int32_t* offsets;       /* int32 [num_experts + 1], expert e owns pairs
                                   [offsets[e], offsets[e+1])                  */
  int32_t num_pairs;            /* P = offsets[num_experts]                    */
  int32_t max_rows_per_expert;  /* host upper bound on offsets[e+1]-offsets[e]
                                   (e.g. T for top-k routing); 0 = num_pairs.
                                   The plan is chosen from it without reading
                                   the device offsets.  If an expert exceeds
                                   it: a plan of the small-M kernel alone
                                   without split K takes the expert in row
                                   chunks (correct, slower); a plan with no
                                   kernel for that many rows sets the
                                   expert's output rows to NaN (never left
                                   unwritten)                                  */
  const float* slot_w;          /* ROUTE_SCALE only: float32 [y_rows]          */
  int32_t y_rows;               /* ROUTE_SCALE only: rows of y                 */
  int32_t epilogue;             /* MILO_EPI_*                                  */
  void* y;                      /* output, see MILO_EPI_*                      */
  int32_t path;                 /* MILO_PATH_*                                 */
  int32_t flags;                /* MILO_GEMM_* bits, normally 0                */
} milo_gemm_desc;

/* desc.flags: the low-rank pre-pass of this descriptor has already been
   enqueued (by milo_moe_lowrank_prepass, same workspace, same stream, nothing
   else using the workspace in between); the GEMM call then enqueues only the
   main kernel(s).  Lets a caller time or schedule the two stages separately. */
#define MILO_GEMM_PREPASS_DONE 1

/* Workspace bytes milo_moe_w3a16_lowrank_gemm needs for this descriptor. */
size_t milo_moe_gemm_workspace_bytes(const milo_gemm_desc* desc);

/*
 * The fused routed grouped GEMM.  For every pair i of expert e (rows of x
 * gathered through sorted_pairs when gather_div > 0), and each weight family w:
 *     Y_w[i] = x_i . deq(W_w,e)^T + (x_i . V_w,e^T) . U_w,e^T
 * (with int3 factors, V and U are their dequantized values (q - z) s, each
 * rounded once to fp16 inside the kernels)
 * [talk] MiLo Algorithm (W_out = W_quant + U V) and MiLo Kernel (int3 x fp16
 * GEMM with dequantization fused into the kernel), with deq(q) = (q - z) * s
 * per 64-column group, fp16 activations and fp32 accumulation.  Then the
 * epilogue: NONE stores Y_0 as fp16; SWIGLU stores silu(Y_0) * Y_1 as fp16
 * (silu(u) = u / (1 + exp(-u))); ROUTE_SCALE stores Y_0 * slot_w[s] as fp32
 * into row s = sorted_pairs[i] (rows of y that no pair maps to are not
 * written).  The path (small-M streaming kernel or matrix-core tile kernel)
 * is chosen per expert from its row count on the device unless forced; with
 * MILO_PATH_AUTO the host plans which kernels to launch from
 * max_rows_per_expert, num_pairs and the matrix size (N K), never from the
 * device offsets.  MILO_PATH_DECODE needs max_rows_per_expert <= 32
 * (MILO_ERR_SHAPE otherwise).  The call is capturable into a HIP graph: it
 * allocates, synchronizes and clears nothing.
 *
 * workspace: milo_moe_gemm_workspace_bytes(desc) bytes (may be 0), 256-byte
 *   aligned, scratch only (no initialisation needed, contents undefined after
 *   the call).  Two calls that overlap in time must not share a workspace.
 * Constraints: N % 64 == 0, K % 128 == 0, N, K <= 65536, 1 <= num_experts
 *   <= 256, num_pairs <= 1048576, x/y/U/V/Uq/Usz/Vq/Vsz 16-byte aligned;
 *   for SWIGLU both families have the same N, K, max_rank and lr_format.
 */
int32_t milo_moe_w3a16_lowrank_gemm(const milo_gemm_desc* desc,
                                    void* workspace, size_t ws_bytes,
                                    void* stream);

/*
 * The first stage of milo_moe_w3a16_lowrank_gemm on its own: the per-pair
 * low-rank products t_i = x_i . V_e^T (fp32 accumulation, stored as fp16 in
 * the workspace), [talk] MiLo Algorithm (W_out = W_quant + U V).  Follow it
 * with milo_moe_w3a16_lowrank_gemm on the same descriptor, workspace and
 * stream with MILO_GEMM_PREPASS_DONE set.  Same validation and workspace rules
 * as the GEMM call; a no-op when max_rank == 0 or num_pairs == 0.
 */
int32_t milo_moe_lowrank_prepass(const milo_gemm_desc* desc, void* workspace,
                                 size_t ws_bytes, void* stream);

/*
 * milo_moe_w3a16_lowrank_gemm without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the scratch lives in a static
 * device array of MILO_STATIC_WORKSPACE_BYTES inside the library, one copy
 * per GPU, held until the process ends.  The call allocates nothing (no
 * hipMalloc, no allocating library routine); the caller still owns every
 * input and output.  Same descriptor, validation and results as the
 * workspace call with desc->flags == 0 (other flags: MILO_ERR_ARG).  A
 * descriptor whose workspace (milo_moe_gemm_workspace_bytes) exceeds the
 * static size returns MILO_ERR_WORKSPACE and enqueues nothing.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and
 * must not be issued.  The scratch needs no initialisation (every byte a call
 * reads was written earlier in the same call).
 */
#define MILO_STATIC_WORKSPACE_BYTES (64u << 20)
int32_t milo_moe_w3a16_lowrank_gemm_static(const milo_gemm_desc* desc, void* stream);

/*
 * Weighted combine: out[t][h] = sum over j = 0..slots-1, in that order, of
 * y[t*slots + j][h] (fp32 adds), rounded to fp16 (nearest even).  y already
 * holds the route-weighted slot outputs (MILO_EPI_ROUTE_SCALE).
 * [talk] Background: a token's output is the combination of the outputs of
 * the experts it activates.
 * y   : float32 [T*slots][H];  out : fp16 [T][H].  H % 4 == 0, 16-byte aligned;
 * 1 <= slots <= 16; T * H / 4 at most 0x7F000000 (MILO_ERR_SHAPE otherwise).
 */
int32_t milo_moe_combine(const float* y, int32_t T, int32_t slots, int32_t H,
                         uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MILO_H */
