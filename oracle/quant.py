"""Group-wise asymmetric int3 round-to-nearest quantization (oracle side).

[talk] Background names round-to-nearest (RTN) as the simplest calibration-free
quantizer; MiLo Algorithm and Key Findings describe the weights as int3 with an
asymmetric zero point, and Experimental Setup & Results describes the
compensators as quantized by simple asymmetric linear quantization.  The pages
give no formula; the reading used here (groups of 64 along the input
dimension K, float16 scale and zero point) is:

    per row n and group g of 64 consecutive k:
        lo, hi = min, max of the group (float64)
        s = f16((hi - lo) / 7);   if s == 0: s = 1      (constant group)
        z = f16_sat(-lo / s)                             (zero point in code units)
        q = clip(rint(w / s + z), 0, 7)                  (round half to even)
        dequant(q) = (q - z) * s

s and z are used at their float16-rounded values.
"""
import numpy as np

F16_MAX = 65504.0


def f16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest float16 (ties to even), returned as
    float16.  NumPy converts float64 -> float16 directly (no float32 step)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def f16_sat(x) -> np.ndarray:
    """float16 rounding that saturates at +-65504 instead of overflowing."""
    return f16_rne(np.clip(np.asarray(x, dtype=np.float64), -F16_MAX, F16_MAX))


def f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def quantize_rtn_int3(W, group: int = 64):
    """W: [R][K] real -> (codes uint8 [R][K] in 0..7, scale fp16 [R][K/group],
    zero fp16 [R][K/group])."""
    W = np.asarray(W)
    R, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    Wg = W.astype(np.float64).reshape(R, K // group, group)
    lo = Wg.min(axis=2)
    hi = Wg.max(axis=2)
    s16 = f16_rne((hi - lo) / 7.0)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    s = s16.astype(np.float64)
    z16 = f16_sat(-lo / s)
    z = z16.astype(np.float64)
    q = np.rint(Wg / s[:, :, None] + z[:, :, None])
    q = np.clip(q, 0, 7).astype(np.uint8).reshape(R, K)
    return q, s16, z16


def dequant_int3(codes, scale, zero, group: int = 64) -> np.ndarray:
    """(q - z) * s in float64, with s, z broadcast over their group."""
    codes = np.asarray(codes)
    R, K = codes.shape
    s = np.asarray(scale).astype(np.float64)
    z = np.asarray(zero).astype(np.float64)
    q = codes.astype(np.float64).reshape(R, K // group, group)
    return ((q - z[:, :, None]) * s[:, :, None]).reshape(R, K)
