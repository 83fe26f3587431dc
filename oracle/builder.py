"""Offline compensator construction (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[talk] MiLo Algorithm, "Compensation Generation": after the initial
quantization the residual W - W_quant is decomposed by SVD and the top-R
singular triplets give the low-rank factors U (out x R) and V (R x in).  The
same section: quantization and compensation are then refined iteratively --
W_quant is recomputed from U V and U V from the new residual.

Readings (the pages give no formulas):
* quantizer: the RTN int3 g64 rule of oracle.quant, or the HQQ-style
  zero-point optimization of oracle.hqq (the pages' initial quantizer);
* iteration t = 1..iters:  Wq_t = quantize(W - L_{t-1}) with L_0 = 0;
  R_t = W - deq(Wq_t);  L_t = best rank-r approximation of R_t;
  the output is (Wq_T, L_T);
* factor split: L = U V with U = U_r diag(sqrt(sigma)), V = diag(sqrt(sigma))
  V_r^T (balanced, so neither factor carries the scale alone -- it matters
  when the factors are quantized to int3 afterwards);
* "SVD" of an N x K residual with N, K in the thousands is computed in the
  library by randomized subspace iteration (Halko, Martinsson & Tropp, SIAM
  Review 2011, Algorithm 4.4) with a caller-drawn Gaussian test matrix; the
  oracle has both that algorithm (same test matrix, fp64, Householder QR from
  NumPy) and the exact truncated SVD it approximates.
"""
import numpy as np

from .hqq import quantize_hqq_int3
from .quant import dequant_int3, quantize_rtn_int3


def residual_ref(W, codes, scale, zero, group=64):
    """R = W - deq(codes) in float64."""
    return np.asarray(W, dtype=np.float64) - dequant_int3(codes, scale, zero, group)


def _split(Ur, s, Vr):
    """Balanced factors of Ur diag(s) Vr."""
    root = np.sqrt(s)
    return Ur * root[None, :], root[:, None] * Vr


def exact_lowrank_ref(R, r):
    """Best rank-r approximation (Eckart-Young) by the full SVD:
    returns (U [N][r], V [r][K], sigma [r]) with U V = U_r diag(sigma) V_r^T."""
    R = np.asarray(R, dtype=np.float64)
    if r == 0:
        return np.zeros((R.shape[0], 0)), np.zeros((0, R.shape[1])), np.zeros(0)
    Uf, s, Vt = np.linalg.svd(R, full_matrices=False)
    U, V = _split(Uf[:, :r], s[:r], Vt[:r])
    return U, V, s[:r]


def rsvd_ref(R, r, omega_t, power_iters):
    """Randomized subspace iteration (Halko et al. 2011, Alg. 4.4), float64.
    omega_t: the Gaussian test matrix stored transposed, [l][K] with
    l = r + oversampling.  Steps:
        Y = R Omega;  Q = orth(Y)
        repeat power_iters times:  Z = orth(R^T Q);  Q = orth(R Z)
        B = Q^T R;  B = Ub diag(s) Vt (small SVD);  keep the top r
        U = Q Ub_r diag(sqrt s_r),  V = diag(sqrt s_r) Vt_r
    Returns (U [N][r], V [r][K], sigma [r])."""
    R = np.asarray(R, dtype=np.float64)
    Om = np.asarray(omega_t, dtype=np.float64).T            # [K][l]
    if r == 0:
        return np.zeros((R.shape[0], 0)), np.zeros((0, R.shape[1])), np.zeros(0)
    Q, _ = np.linalg.qr(R @ Om)
    for _ in range(power_iters):
        Z, _ = np.linalg.qr(R.T @ Q)
        Q, _ = np.linalg.qr(R @ Z)
    B = Q.T @ R
    Ub, s, Vt = np.linalg.svd(B, full_matrices=False)
    U, V = _split(Q @ Ub[:, :r], s[:r], Vt[:r])
    return U, V, s[:r]


def build_ref(W, r, iters, omegas_t, power_iters, group=64, quantizer="rtn"):
    """The refinement loop above with the randomized SVD; omegas_t[t] is the
    test matrix of iteration t ([iters][l][K]).  Returns a dict with the last
    codes/scale/zero, U, V, sigma, and the per-iteration errors
    ||W - deq(Wq_t) - L_t||_F and ||W - deq(Wq_t)||_F."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    L = np.zeros_like(W)
    U = np.zeros((N, r))
    V = np.zeros((r, K))
    sigma = np.zeros(r)
    errs, res_norms = [], []
    codes = scale = zero = None
    for t in range(iters):
        quantize = quantize_hqq_int3 if quantizer == "hqq" else quantize_rtn_int3
        codes, scale, zero = quantize(W - L, group)
        R = residual_ref(W, codes, scale, zero, group)
        U, V, sigma = rsvd_ref(R, r, omegas_t[t], power_iters)
        L = U @ V
        res_norms.append(float(np.linalg.norm(R)))
        errs.append(float(np.linalg.norm(R - L)))
    return {"codes": codes, "scale": scale, "zero": zero, "U": U, "V": V, "sigma": sigma,
            "errors": errs, "residual_norms": res_norms}
