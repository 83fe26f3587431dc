"""The validity checks of tests/int_checks.py (used by the GPU parity tests
of the quantizers and the compensator builder) accept the oracle's own
outputs and reject planted mistakes that are not rounding ties."""
import numpy as np
import pytest

import oracle
from oracle import hqq as HQ
from tests import int_checks as IC


def _w(R, K, seed, scale=0.02):
    return (np.random.default_rng(seed).standard_normal((R, K)) * scale).astype(np.float32)


def test_near_f16_midpoint():
    # 1 + 2^-11 is the midpoint between 1 and the next float16 (1 + 2^-10)
    assert IC.near_f16_midpoint(np.array([1.0 + 2.0 ** -11]), 1e-9)[0]
    assert not IC.near_f16_midpoint(np.array([1.0 + 2.0 ** -12]), 1e-9)[0]
    assert not IC.near_f16_midpoint(np.array([1.0]), 1e-9)[0]


def test_rtn_check_accepts_oracle_and_rejects_mistakes():
    W = _w(64, 256, 1).astype(np.float64)
    q, s, z = oracle.quantize_rtn_int3(W)
    assert IC.assert_rtn_valid(W, q, s, z, 1e-9, 1e-9, "oracle") == (0, 0)
    bad = q.copy()
    # a code moved by one level at a weight far from a tie
    t = W / np.repeat(s.astype(np.float64), 64, axis=1) + np.repeat(z.astype(np.float64), 64, axis=1)
    i, j = np.argwhere(np.abs(t - np.floor(t) - 0.5) > 0.2)[0]
    bad[i, j] = bad[i, j] + 1 if bad[i, j] < 7 else bad[i, j] - 1
    with pytest.raises(AssertionError):
        IC.assert_rtn_valid(W, bad, s, z, 1e-9, 1e-9, "planted code")
    zb = z.copy()
    zb[3, 1] = np.float16(float(zb[3, 1]) + 0.25)
    with pytest.raises(AssertionError):
        IC.assert_rtn_valid(W, q, s, zb, 1e-9, 1e-9, "planted zero")
    sb = s.copy()
    sb[5, 2] = np.float16(float(sb[5, 2]) * 1.01)
    with pytest.raises(AssertionError):
        IC.assert_rtn_valid(W, q, sb, z, 1e-9, 1e-9, "planted scale")


def test_rtn_check_excuses_a_tie():
    # one group with a weight exactly on a rounding tie: either code is valid
    W = np.zeros((1, 64))
    W[0, 0], W[0, 1] = 0.0, 7.0
    W[0, 2] = 2.5                                   # s = 1, z = 0: w/s + z = 2.5
    q, s, z = oracle.quantize_rtn_int3(W)
    alt = q.copy()
    alt[0, 2] = 3 if q[0, 2] == 2 else 2
    assert IC.assert_rtn_valid(W, alt, s, z, 1e-9, 1e-9, "tie")[1] == 1


def test_hqq_check_accepts_oracle_and_rejects_mistakes():
    W = _w(32, 512, 2, 1.0).astype(np.float64)        # unit scale: the threshold is active
    c, s, z = HQ.quantize_hqq_int3(W)
    assert IC.assert_hqq_valid(W, c, s, z, "oracle") == 0
    # a zero point replaced by the RTN one where that is strictly worse
    _, _, z0 = oracle.quantize_rtn_int3(W)
    w = W.reshape(32, 8, 64)
    s3 = s.astype(np.float64)[..., None]
    e_h = HQ.group_mae(w, s3, z.astype(np.float64)[..., None])
    e_r = HQ.group_mae(w, s3, z0.astype(np.float64)[..., None])
    i, j = np.argwhere(e_h < e_r * (1 - 1e-6))[0]
    zb, cb = z.copy(), c.copy()
    zb[i, j] = z0[i, j]
    cb.reshape(32, 8, 64)[i, j] = np.clip(np.rint(w[i, j] / float(s[i, j]) + float(z0[i, j])), 0, 7)
    with pytest.raises(AssertionError):
        IC.assert_hqq_valid(W, cb, s, zb, "planted zero point")
    # codes not taken at the stored zero point
    cb = c.copy()
    cb.reshape(32, 8, 64)[0, 0, :] = np.clip(cb.reshape(32, 8, 64)[0, 0, :].astype(int) + 1, 0, 7)
    with pytest.raises(AssertionError):
        IC.assert_hqq_valid(W, cb, s, z, "planted codes")
