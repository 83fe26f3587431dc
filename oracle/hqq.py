"""HQQ-style int3 quantizer (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[talk] Key Findings and MiLo Algorithm: MiLo's initial quantization is HQQ,
which needs no calibration data; the pages give neither its objective nor its
solver.  The published method (Badri & Shaji, "Half-Quadratic Quantization of
Large Machine Learning Models", 2023) keeps the min-max scale and optimizes
the zero point of each group for a sparsity-promoting l_p error (p < 1) by
half-quadratic splitting: with an auxiliary error variable W_e,

    q    = clip(rint(w / s + z), 0, 7)            quantize with the current z
    W_e  = shrink_p(w - (q - z) s, beta)          generalized soft threshold:
           shrink_p(x) = sign(x) max(|x| - |x|^(p-1) / beta, 0)
    z    = mean over the group of (q - (w - W_e) / s)   closed-form zero update
    beta = kappa beta

Readings used here (parity of the method: unpinned; only the mechanics and
the no-worse-than-RTN guarantee below are pinned):
* start from the RTN g64 parameters of oracle.quant (same fp16 scale; zero
  point z_0 = its fp16 zero);
* a fixed number of iterations (defaults p = 0.7, beta = 10, kappa = 1.01,
  20 iterations -- the method's published defaults); z evolves unrounded;
* after every iteration the candidate fp16 zero point f16(z) is scored by the
  group's mean absolute error with codes chosen at that zero point, and each
  group keeps its best candidate (the RTN zero point is candidate 0), so no
  group is ever worse than RTN by that measure;
* the stored codes are rint(w / s + z*) clipped, with the kept fp16 z*.
"""
import numpy as np

from .quant import f16_sat, quantize_rtn_int3


def shrink_lp(x, beta, p):
    """sign(x) * max(|x| - |x|^(p-1) / beta, 0), with shrink(0) = 0."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        t = ax - np.power(ax, p - 1.0) / beta
    return np.sign(x) * np.maximum(t, 0.0)


def _codes(w, s, z):
    return np.clip(np.rint(w / s + z), 0.0, 7.0)


def group_mae(w, s, z):
    """Mean |w - deq| over the last axis for codes chosen at zero point z."""
    return np.mean(np.abs(w - (_codes(w, s, z) - z) * s), axis=-1)


def hqq_zero_step(w, s, z, beta, p):
    """One half-quadratic update of the zero point of each group (last axis):
    returns the new (unrounded) z, shape of z."""
    q = _codes(w, s, z)
    we = shrink_lp(w - (q - z) * s, beta, p)
    return np.mean(q - (w - we) / s, axis=-1, keepdims=True)


def hqq_zero_trajectory(w, s, z0, iters, p=0.7, beta=10.0, kappa=1.01):
    """The unrounded zero points z_1 .. z_iters of the half-quadratic
    iteration started at z0 (w: [..., group], s and z0: [..., 1]); the
    threshold parameter is beta at the first update and grows by the factor
    kappa after each one.  Returns a list of arrays shaped like z0."""
    z = np.asarray(z0, dtype=np.float64)
    out = []
    b = float(beta)
    for _ in range(iters):
        z = hqq_zero_step(w, s, z, b, p)
        b *= kappa
        out.append(z)
    return out


def quantize_hqq_int3(W, group=64, iters=20, p=0.7, beta=10.0, kappa=1.01):
    """W [R][K] -> (codes uint8 [R][K], scale fp16 [R][K/group], zero fp16
    [R][K/group]); scale is the RTN scale."""
    W = np.asarray(W)
    R, K = W.shape
    _, s16, z16 = quantize_rtn_int3(W, group)
    w = W.astype(np.float64).reshape(R, K // group, group)
    s = s16.astype(np.float64)[..., None]
    z0 = z16.astype(np.float64)[..., None]
    best = z0.copy()
    best_err = group_mae(w, s, best)
    for z in hqq_zero_trajectory(w, s, z0, iters, p, beta, kappa):
        zc = f16_sat(z).astype(np.float64)
        err = group_mae(w, s, zc)
        better = err < best_err
        best = np.where(better[..., None], zc, best)
        best_err = np.where(better, err, best_err)
    codes = _codes(w, s, best).astype(np.uint8).reshape(R, K)
    return codes, s16, best[..., 0].astype(np.float16)
