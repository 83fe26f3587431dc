// Offline compensator construction on the GPU: residual of the int3
// quantization, its rank-r approximation by randomized subspace iteration,
// and the quantize <-> compensate refinement.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), MiLo Algorithm, "Compensation
// Generation": the residual W - W_quant is decomposed by SVD and its top-R
// singular triplets give the factors U (out x R) and V (R x in); W_quant and
// U V are then refined in turn.  The truncated SVD of an N x K residual is
// computed by randomized subspace iteration (Halko, Martinsson & Tropp,
// "Finding structure with randomness", SIAM Review 2011, Algorithm 4.4) with a
// Gaussian test matrix drawn by the caller:
//     Y = R Omega;  Q = orth(Y);  repeat q times: Z = orth(R^T Q), Q = orth(R Z)
//     B = Q^T R;  B B^T = W diag(lambda) W^T;  keep the top r
//     U = Q W_r diag(sigma^(1/2)),  V = diag(sigma^(-1/2)) W_r^T B,  sigma = lambda^(1/2)
// so that U V = Q W_r W_r^T Q^T R is the rank-r approximation and the factors
// are balanced (column norms of U = row norms of V = sigma^(1/2)).
// orth() is CholeskyQR2 (Gram matrix, Cholesky, triangular solve, twice).
//
// The big products are tall-and-skinny fp32 GEMMs with one dimension l =
// r + oversampling <= 80: gemm_nt (Y = A X^T, each block 64 rows of A x all l
// outputs, tiles staged through LDS) and gemm_tn (C = A^T B, reduction over
// rows split across blocks, partial sums added in split order).  The l x l
// factorizations (Cholesky, symmetric eigenproblem by parallel-ordered Jacobi
// rotations) run in one block in fp64 in LDS.  Deterministic throughout.
#include "milo_internal.hpp"

namespace milo {

constexpr int kMaxL = 80;          // rank + oversampling
// HQQ settings of the refinement (the method's published defaults)
constexpr int kHqqIters = 20;
constexpr double kHqqP = 0.7, kHqqBeta = 10.0, kHqqKappa = 1.01;
constexpr int kSplitRows = 512;    // target rows per gemm_tn split

// ---------------------------------------------------------------- elementwise

// R = W - (q - z) s, per 64-column group; exact product, one rounding.
__global__ void __launch_bounds__(256) residual_kernel(const float* __restrict__ W,
                                                       const uint8_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ scale,
                                                       const uint16_t* __restrict__ zero,
                                                       int64_t N, int64_t K, float* __restrict__ R) {
  const int64_t n = N * K, groups = K / kGroup;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / K, g = (i - row * K) / kGroup;
    const float s = half_bits_to_float(scale[row * groups + g]);
    const float z = half_bits_to_float(zero[row * groups + g]);
    R[i] = __builtin_fmaf(-((float)codes[i] - z), s, W[i]);
  }
}

// out = W - U V for U [N][r], V [r][K]: 64 x 64 output tile per block, both
// factor tiles in LDS, 4 x 4 outputs per thread.
__global__ void __launch_bounds__(256) lowrank_sub_kernel(const float* __restrict__ W,
                                                          const float* __restrict__ U,
                                                          const float* __restrict__ V, int64_t N,
                                                          int64_t K, int r, float* __restrict__ out) {
  __shared__ float us[64][65];
  __shared__ float vs[64][65];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int64_t n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
  for (int i = t; i < 64 * 64; i += 256) {
    const int a = i >> 6, b = i & 63;
    us[a][b] = (n0 + a < N && b < r) ? U[(n0 + a) * r + b] : 0.f;       // us[row][j]
    vs[a][b] = (a < r && k0 + b < K) ? V[a * K + k0 + b] : 0.f;         // vs[j][col]
  }
  __syncthreads();
  float acc[4][4] = {};
  for (int j = 0; j < r; ++j) {
    float uu[4], vv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) uu[a] = us[4 * ty + a][j];
#pragma unroll
    for (int b = 0; b < 4; ++b) vv[b] = vs[j][4 * tx + b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(uu[a], vv[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t n = n0 + 4 * ty + a;
    if (n >= N) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t k = k0 + 4 * tx + b;
      if (k < K) out[n * K + k] = W[n * K + k] - acc[a][b];
    }
  }
}

// ---------------------------------------------------------------- skinny GEMMs

// Y[n][j] = sum_k A[n][k] Xt[j][k]  (n < Nr, j < lj <= kMaxL, k < Kd).
// Block: 64 rows; thread (rg = t mod 16, jg = t div 16) owns rows 4 rg .. +3
// and outputs j = jg + 16 i.  K in chunks of 32 through LDS.
// With gridDim.y > 1 the K range is split: block y covers
// [y k_per_split, (y + 1) k_per_split) and stores its partial sums at
// Y + y Nr ldy (summed afterwards in split order).
__global__ void __launch_bounds__(256) gemm_nt_kernel(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ Xt, int64_t ldx,
                                                      float* __restrict__ Y, int64_t ldy, int64_t Nr,
                                                      int64_t Kd, int lj, int64_t k_per_split) {
  constexpr int KC = 32, JI = kMaxL / 16;
  __shared__ float as[64][KC + 1];
  __shared__ float xs[kMaxL][KC + 1];
  const int t = threadIdx.x, rg = t & 15, jg = t >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t kA = (int64_t)blockIdx.y * k_per_split;
  const int64_t kB = kA + k_per_split < Kd ? kA + k_per_split : Kd;
  Y += (size_t)blockIdx.y * Nr * ldy;
  float acc[4][JI] = {};
  for (int64_t k0 = kA; k0 < kB; k0 += KC) {
    for (int i = t; i < 64 * KC; i += 256) {
      const int a = i / KC, kk = i - a * KC;
      as[a][kk] = (n0 + a < Nr && k0 + kk < kB) ? A[(n0 + a) * lda + k0 + kk] : 0.f;
    }
    for (int i = t; i < lj * KC; i += 256) {
      const int j = i / KC, kk = i - j * KC;
      xs[j][kk] = (k0 + kk < kB) ? Xt[j * ldx + k0 + kk] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < KC; ++kk) {
      float av[4], xv[JI];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = as[4 * rg + a][kk];
#pragma unroll
      for (int i = 0; i < JI; ++i) xv[i] = (jg + 16 * i < lj) ? xs[jg + 16 * i][kk] : 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < JI; ++i) acc[a][i] = __builtin_fmaf(av[a], xv[i], acc[a][i]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t n = n0 + 4 * rg + a;
    if (n >= Nr) continue;
#pragma unroll
    for (int i = 0; i < JI; ++i)
      if (jg + 16 * i < lj) Y[n * ldy + jg + 16 * i] = acc[a][i];
  }
}

// part[s][a][b] = sum over rows n of split s of A[n][a] B[n][b]
// (a < la <= kMaxL, b < lb).  Block: 64 columns of B x all a; thread
// (cg = t mod 16, ag = t div 16) owns columns 4 cg .. +3 and a = ag + 16 i.
// Rows in chunks of 32 through LDS.
__global__ void __launch_bounds__(256) gemm_tn_kernel(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ B, int64_t ldb,
                                                      float* __restrict__ part, int64_t Nr, int la,
                                                      int64_t lb, int64_t rows_per_split) {
  constexpr int NC = 32, AI = kMaxL / 16;
  __shared__ float as[NC][kMaxL + 1];
  __shared__ float bs[NC][64 + 1];
  const int t = threadIdx.x, cg = t & 15, ag = t >> 4;
  const int64_t b0 = (int64_t)blockIdx.x * 64;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < Nr ? r0 + rows_per_split : Nr;
  float acc[AI][4] = {};
  for (int64_t c0 = r0; c0 < r1; c0 += NC) {
    for (int i = t; i < NC * la; i += 256) {
      const int n = i / la, a = i - n * la;
      as[n][a] = (c0 + n < r1) ? A[(c0 + n) * lda + a] : 0.f;
    }
    for (int i = t; i < NC * 64; i += 256) {
      const int n = i >> 6, b = i & 63;
      bs[n][b] = (c0 + n < r1 && b0 + b < lb) ? B[(c0 + n) * ldb + b0 + b] : 0.f;
    }
    __syncthreads();
    for (int n = 0; n < NC; ++n) {
      float av[AI], bv[4];
#pragma unroll
      for (int i = 0; i < AI; ++i) av[i] = (ag + 16 * i < la) ? as[n][ag + 16 * i] : 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = bs[n][4 * cg + b];
#pragma unroll
      for (int i = 0; i < AI; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[i][b] = __builtin_fmaf(av[i], bv[b], acc[i][b]);
    }
    __syncthreads();
  }
  float* out = part + (size_t)blockIdx.y * la * lb;
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int a = ag + 16 * i;
    if (a >= la) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t c = b0 + 4 * cg + b;
      if (c < lb) out[(size_t)a * lb + c] = acc[i][b];
    }
  }
}

// C[i] = sum over splits, in split order, of part[s][i].
__global__ void __launch_bounds__(256) sum_splits_kernel(const float* __restrict__ part, int nsplit,
                                                         int64_t n, float* __restrict__ C) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < nsplit; ++s) v += part[(size_t)s * n + i];
    C[i] = v;
  }
}

// ---------------------------------------------------------------- l x l factorizations (one block, fp64)

// Cholesky G = L L^T of a symmetric positive semi-definite l x l matrix and
// the inverse of L.  A pivot at or below 1e-12 of the largest diagonal entry
// marks its direction dead: that row of L^-1 is zero, so the matching column
// of the orthonormalized block is zero (rank-deficient or zero input).
// Outputs Linv [l][l] and its transpose (fp32).
__global__ void __launch_bounds__(256) small_chol_kernel(const float* __restrict__ G, int l,
                                                         float* __restrict__ Linv,
                                                         float* __restrict__ LinvT) {
  __shared__ double A[kMaxL][kMaxL + 1];   // G, then L in the lower triangle
  __shared__ double X[kMaxL][kMaxL + 1];   // L^-1
  __shared__ int dead[kMaxL];
  __shared__ double gmax;
  const int t = threadIdx.x;
  for (int i = t; i < l * l; i += blockDim.x) {
    A[i / l][i % l] = (double)G[i];
    X[i / l][i % l] = (i / l == i % l) ? 1.0 : 0.0;
  }
  __syncthreads();
  if (t < 64) {                              // largest diagonal entry (one wave)
    double m = 0.0;
    for (int i = t; i < l; i += 64) m = fmax(m, A[i][i]);
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o));
    if (t == 0) gmax = m;
  }
  __syncthreads();
  // right-looking: pivot, scale the column, update the trailing triangle
  // (every step's work is spread over the block; nothing serial but the pivot)
  for (int j = 0; j < l; ++j) {
    if (t == 0) {
      const double d = A[j][j];
      const bool dd = !(d > 1e-12 * gmax) || !(gmax > 0.0);
      dead[j] = dd;
      A[j][j] = dd ? 1.0 : sqrt(d);
    }
    __syncthreads();
    const double piv = A[j][j];
    for (int i = j + 1 + t; i < l; i += blockDim.x) A[i][j] = dead[j] ? 0.0 : A[i][j] / piv;
    __syncthreads();
    // 16 x 16 thread grid over (i, k): no integer division in the loops
    for (int i = j + 1 + (t >> 4); i < l; i += 16)
      for (int k = j + 1 + (t & 15); k <= i; k += 16) A[i][k] -= A[i][j] * A[k][j];
    __syncthreads();
  }
  // X = L^-1 by the same right-looking pattern: row i is final once divided
  // by L[i][i]; it is then eliminated from every later row
  for (int i = 0; i < l; ++i) {
    const double piv = A[i][i];
    for (int c = t; c <= i; c += blockDim.x) X[i][c] /= piv;
    __syncthreads();
    for (int k = i + 1 + (t >> 4); k < l; k += 16)
      for (int c = (t & 15); c <= i; c += 16) X[k][c] -= A[k][i] * X[i][c];
    __syncthreads();
  }
  for (int i = t; i < l * l; i += blockDim.x) {
    const int a = i / l, b = i % l;
    const double v = dead[a] ? 0.0 : X[a][b];
    Linv[a * l + b] = (float)v;
    LinvT[b * l + a] = (float)v;
  }
}

// Symmetric eigenproblem of the l x l matrix Gb = B B^T by two-sided Jacobi
// rotations in parallel (round-robin) order, fp64, then the top r of the
// eigenpairs (descending): sigma_i = sqrt(max(lambda_i, 0)),
// XtU[i][j] = w_j,i sigma_i^(1/2)  (U = Q XtU^T), AV[j][i] = w_j,i sigma_i^(-1/2)
// (V = AV^T B; zero where sigma_i = 0).  l is padded to an even size with a
// zero row and column.
__global__ void __launch_bounds__(256) small_eig_kernel(const float* __restrict__ Gb, int l, int r,
                                                        float* __restrict__ XtU, float* __restrict__ AV,
                                                        float* __restrict__ sigma) {
  __shared__ double S[kMaxL][kMaxL + 1];
  __shared__ double Wm[kMaxL][kMaxL + 1];
  __shared__ double cs[kMaxL / 2], sn[kMaxL / 2];
  __shared__ int pp[kMaxL / 2], qq[kMaxL / 2];
  __shared__ int order[kMaxL];
  __shared__ double off_sum, diag_sum;
  const int t = threadIdx.x;
  const int n = (l + 1) & ~1;
  for (int i = t; i < n * n; i += blockDim.x) {
    const int a = i / n, b = i % n;
    S[a][b] = (a < l && b < l) ? (double)Gb[a * l + b] : 0.0;
    Wm[a][b] = (a == b) ? 1.0 : 0.0;
  }
  __syncthreads();
  __shared__ double red_o[256], red_d[256];
  for (int sweep = 0; sweep < 30; ++sweep) {
    // off-diagonal and diagonal energy, block reduction in a fixed order
    double o = 0.0, d = 0.0;
    for (int a = t >> 6; a < n; a += 4)
      for (int b = t & 63; b < n; b += 64) {
        const double v = S[a][b] * S[a][b];
        if (a == b) d += v;
        else o += v;
      }
    red_o[t] = o;
    red_d[t] = d;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (t < w) {
        red_o[t] += red_o[t + w];
        red_d[t] += red_d[t + w];
      }
      __syncthreads();
    }
    if (t == 0) {
      off_sum = red_o[0];
      diag_sum = red_d[0];
    }
    __syncthreads();
    // stop once the off-diagonal norm is below 1e-11 of the diagonal norm (the
    // rounding floor of the rotations is about 1e-14 of the largest entry)
    if (!(off_sum > 1e-22 * diag_sum)) break;
    for (int step = 0; step < n - 1; ++step) {
      // pairs of this step: (n-1, step), ((step + i) mod (n-1), (step - i) mod (n-1))
      for (int i = t; i < n / 2; i += blockDim.x) {
        int p, q;
        if (i == 0) {
          p = n - 1;
          q = step;
        } else {
          p = (step + i) % (n - 1);
          q = (step - i + (n - 1)) % (n - 1);
        }
        if (p > q) {
          const int tmp = p;
          p = q;
          q = tmp;
        }
        const double apq = S[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (S[q][q] - S[p][p]) / (2.0 * apq);
          const double tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + tt * tt);
          s = tt * c;
        }
        pp[i] = p;
        qq[i] = q;
        cs[i] = c;
        sn[i] = s;
      }
      __syncthreads();
      // rows: S <- J^T S (each pair rotates its two rows, all columns);
      // thread (t div 64, t mod 64) walks pairs by 4 and columns by 64
      for (int i = t >> 6; i < n / 2; i += 4)
        for (int col = t & 63; col < n; col += 64) {
          const int p = pp[i], q = qq[i];
          const double c = cs[i], s = sn[i];
          const double sp = S[p][col], sq = S[q][col];
          S[p][col] = c * sp - s * sq;
          S[q][col] = s * sp + c * sq;
        }
      __syncthreads();
      // columns: S <- S J, and W <- W J
      for (int i = t >> 6; i < n / 2; i += 4)
        for (int row = t & 63; row < n; row += 64) {
          const int p = pp[i], q = qq[i];
          const double c = cs[i], s = sn[i];
          const double sp = S[row][p], sq = S[row][q];
          S[row][p] = c * sp - s * sq;
          S[row][q] = s * sp + c * sq;
          const double wp = Wm[row][p], wq = Wm[row][q];
          Wm[row][p] = c * wp - s * wq;
          Wm[row][q] = s * wp + c * wq;
        }
      __syncthreads();
    }
  }
  // order: descending eigenvalue, ties by index (stable selection by rank)
  for (int a = t; a < n; a += blockDim.x) {
    int rank = 0;
    for (int b = 0; b < n; ++b)
      if (S[b][b] > S[a][a] || (S[b][b] == S[a][a] && b < a)) ++rank;
    order[rank] = a;
  }
  __syncthreads();
  for (int idx = t; idx < r * l; idx += blockDim.x) {
    const int i = idx / l, j = idx % l;
    const int col = order[i];
    const double lam = S[col][col] > 0.0 ? S[col][col] : 0.0;
    const double sg = sqrt(lam), rt = sqrt(sg);
    const double w = Wm[j][col];
    XtU[i * l + j] = (float)(w * rt);
    AV[j * r + i] = rt > 0.0 ? (float)(w / rt) : 0.f;
    if (j == 0) sigma[i] = (float)sg;
  }
}

// ---------------------------------------------------------------- host orchestration

static int grid_1d(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

struct SvdWs {
  float *Y, *Y2, *Bm, *Bm2, *part, *G, *Linv, *LinvT, *XtU, *AV;
  int nsplit;
};

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

static int tn_splits(int64_t Nr) {
  int64_t s = (Nr + kSplitRows - 1) / kSplitRows;
  return (int)(s < 1 ? 1 : (s > 64 ? 64 : s));
}

size_t svd_workspace_bytes(int64_t N, int64_t K, int l) {
  const int64_t big = N > K ? N : K;
  const int ns = tn_splits(N > K ? N : K);
  size_t b = 0;
  b += 2 * align256((size_t)N * l * 4);                 // Y, Y2
  b += 2 * align256((size_t)l * K * 4);                 // Bm, Bm2
  b += align256((size_t)ns * l * (big > l ? big : l) * 4);  // partial sums
  b += 5 * align256((size_t)kMaxL * kMaxL * 4);         // G, Linv, LinvT, XtU, AV
  return b;
}

static SvdWs carve(char* ws, int64_t N, int64_t K, int l) {
  SvdWs w;
  const int64_t big = N > K ? N : K;
  w.nsplit = tn_splits(big);
  char* p = ws;
  auto take = [&](size_t bytes) {
    float* f = (float*)p;
    p += align256(bytes);
    return f;
  };
  w.Y = take((size_t)N * l * 4);
  w.Y2 = take((size_t)N * l * 4);
  w.Bm = take((size_t)l * K * 4);
  w.Bm2 = take((size_t)l * K * 4);
  w.part = take((size_t)w.nsplit * l * (big > l ? big : l) * 4);
  w.G = take(kMaxL * kMaxL * 4);
  w.Linv = take(kMaxL * kMaxL * 4);
  w.LinvT = take(kMaxL * kMaxL * 4);
  w.XtU = take(kMaxL * kMaxL * 4);
  w.AV = take(kMaxL * kMaxL * 4);
  return w;
}

// Y [Nr][lj] = A [Nr][Kd] Xt^T; K split over blocks (partials in the
// workspace, summed in split order) until about 1024 blocks run.
static void nt(const float* A, int64_t lda, const float* Xt, int64_t ldx, float* Y, int64_t ldy,
               int64_t Nr, int64_t Kd, int lj, const SvdWs& w, hipStream_t st) {
  const int64_t tiles = (Nr + 63) / 64;
  int64_t ks = 1024 / tiles;
  const int64_t ks_max = Kd / 64;                   // at least 64 columns per split
  if (ks > ks_max) ks = ks_max;
  if (ks > w.nsplit) ks = w.nsplit;
  if (ldy != lj) ks = 1;                            // partials are packed [Nr][lj]
  if (ks <= 1) {
    hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)tiles, 1), dim3(256), 0, st, A, lda, Xt, ldx, Y, ldy, Nr,
                       Kd, lj, Kd);
    return;
  }
  int64_t kps = (Kd + ks - 1) / ks;
  kps = (kps + 31) / 32 * 32;
  ks = (Kd + kps - 1) / kps;
  hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)tiles, (unsigned)ks), dim3(256), 0, st, A, lda, Xt, ldx,
                     w.part, (int64_t)lj, Nr, Kd, lj, kps);
  const int64_t n = Nr * lj;
  hipLaunchKernelGGL(sum_splits_kernel, dim3(grid_1d(n)), dim3(256), 0, st, w.part, (int)ks, n, Y);
}

// C [la][lb] = A^T B, A [Nr][la], B [Nr][lb]
static void tn(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t Nr, int la,
               int64_t lb, const SvdWs& w, hipStream_t st) {
  int ns = tn_splits(Nr);
  if (ns > w.nsplit) ns = w.nsplit;
  const int64_t rps = (Nr + ns - 1) / ns;
  hipLaunchKernelGGL(gemm_tn_kernel, dim3((unsigned)((lb + 63) / 64), ns), dim3(256), 0, st, A, lda, B, ldb,
                     w.part, Nr, la, lb, rps);
  const int64_t n = (int64_t)la * lb;
  hipLaunchKernelGGL(sum_splits_kernel, dim3(grid_1d(n)), dim3(256), 0, st, w.part, ns, n, C);
}

// Orthonormal columns of Y [Nr][l] in place (CholeskyQR2), using Y2.
static void orth_rows(float* Y, float* Y2, int64_t Nr, int l, const SvdWs& w, hipStream_t st) {
  for (int pass = 0; pass < 2; ++pass) {
    float* src = pass == 0 ? Y : Y2;
    float* dst = pass == 0 ? Y2 : Y;
    tn(src, l, src, l, w.G, Nr, l, l, w, st);
    hipLaunchKernelGGL(small_chol_kernel, dim3(1), dim3(256), 0, st, w.G, l, w.Linv, w.LinvT);
    nt(src, l, w.Linv, l, dst, l, Nr, l, l, w, st);   // dst = src L^-T
  }
}

// Orthonormal rows of Zt [l][K] in place (CholeskyQR2 of Z = Zt^T), using Z2t.
static void orth_cols(float* Zt, float* Z2t, int64_t K, int l, const SvdWs& w, hipStream_t st) {
  for (int pass = 0; pass < 2; ++pass) {
    float* src = pass == 0 ? Zt : Z2t;
    float* dst = pass == 0 ? Z2t : Zt;
    nt(src, K, src, K, w.G, l, l, K, l, w, st);       // G = Zt Zt^T
    hipLaunchKernelGGL(small_chol_kernel, dim3(1), dim3(256), 0, st, w.G, l, w.Linv, w.LinvT);
    tn(w.LinvT, l, src, K, dst, l, l, K, w, st);      // dst = L^-1 Zt  (LinvT^T = L^-1)
  }
}

int32_t run_lowrank_svd(const float* R, int64_t N, int64_t K, int r, int l, int q, const float* omega_t,
                        float* U, float* V, float* sigma, char* ws, hipStream_t st) {
  SvdWs w = carve(ws, N, K, l);
  nt(R, K, omega_t, K, w.Y, l, N, K, l, w, st);       // Y = R Omega
  orth_rows(w.Y, w.Y2, N, l, w, st);
  for (int i = 0; i < q; ++i) {
    tn(w.Y, l, R, K, w.Bm, N, l, K, w, st);           // Z^T = Q^T R
    orth_cols(w.Bm, w.Bm2, K, l, w, st);
    nt(R, K, w.Bm, K, w.Y, l, N, K, l, w, st);        // Y = R Z
    orth_rows(w.Y, w.Y2, N, l, w, st);
  }
  tn(w.Y, l, R, K, w.Bm, N, l, K, w, st);             // B = Q^T R
  nt(w.Bm, K, w.Bm, K, w.G, l, l, K, l, w, st);       // B B^T
  hipLaunchKernelGGL(small_eig_kernel, dim3(1), dim3(256), 0, st, w.G, l, r, w.XtU, w.AV, sigma);
  nt(w.Y, l, w.XtU, l, U, r, N, l, r, w, st);         // U = Q W_r sigma^(1/2)
  tn(w.AV, r, w.Bm, K, V, l, r, K, w, st);            // V = sigma^(-1/2) W_r^T B
  return hip_status(hipGetLastError(), "lowrank svd launches");
}

size_t build_workspace_bytes(int64_t N, int64_t K, int l) {
  return align256((size_t)N * K * 4) + svd_workspace_bytes(N, K, l);
}

int32_t run_build(const float* W, int64_t N, int64_t K, int r, int iters, int l, int q, const float* omega,
                  int quantizer, uint8_t* codes, uint16_t* scale, uint16_t* zero, float* U, float* V,
                  float* sigma, char* ws, hipStream_t st) {
  float* Rm = (float*)ws;
  char* svd_ws = ws + align256((size_t)N * K * 4);
  for (int it = 0; it < iters; ++it) {
    const float* target = W;
    if (it > 0 && r > 0) {
      hipLaunchKernelGGL(lowrank_sub_kernel, dim3((unsigned)((K + 63) / 64), (unsigned)((N + 63) / 64)),
                         dim3(256), 0, st, W, U, V, N, K, r, Rm);
      target = Rm;
    }
    int32_t rc = quantizer == MILO_QUANT_HQQ
                     ? launch_hqq(target, N, K, kHqqIters, kHqqP, kHqqBeta, kHqqKappa, codes, scale, zero, st)
                     : launch_quantize(target, N, K, kGroup, codes, scale, zero, st);
    if (rc != MILO_OK) return rc;
    if (r == 0) continue;
    hipLaunchKernelGGL(residual_kernel, dim3(grid_1d(N * K)), dim3(256), 0, st, W, codes, scale, zero, N, K,
                       Rm);
    rc = run_lowrank_svd(Rm, N, K, r, l, q, omega + (size_t)it * l * K, U, V, sigma, svd_ws, st);
    if (rc != MILO_OK) return rc;
  }
  return hip_status(hipGetLastError(), "compensator build launches");
}

}  // namespace milo
