"""Pins for the oracle's HQQ-style quantizer (oracle/hqq.py).  The method's
objective and solver are not on the pages (parity of the method: unpinned);
pinned here are the operator and the update in closed form, the start and
limits, and the guarantee the reading adds: no group worse than RTN."""
import numpy as np
import pytest

import oracle
from oracle import hqq as HQ


def test_shrink_closed_forms():
    x = np.array([0.0, 4.0, -4.0, 0.25, -0.25, 1.0])
    got = HQ.shrink_lp(x, 1.0, 0.5)          # |x| - |x|^(-1/2), clipped at 0, sign kept
    np.testing.assert_allclose(got, [0.0, 3.5, -3.5, 0.0, 0.0, 0.0], rtol=0, atol=1e-15)
    assert HQ.shrink_lp(np.array([9.0]), 2.0, 0.5)[0] == pytest.approx(9.0 - (1.0 / 3.0) / 2.0)


def _w(R, K, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "heavy":
        return (rng.standard_t(3, (R, K)) * 0.02).astype(np.float32)
    if kind == "wide":
        return rng.standard_normal((R, K)).astype(np.float32)
    return (rng.standard_normal((R, K)) * 0.02).astype(np.float32)


def test_zero_update_limits():
    """beta -> infinity: the error variable absorbs everything and the zero
    point stays put; beta -> 0: no error variable, and the update is the
    least-squares zero point for the current codes, mean(q - w / s)."""
    W = _w(8, 128, 1)
    q, s16, z16 = oracle.quantize_rtn_int3(W)
    w = W.astype(np.float64).reshape(8, 2, 64)
    s = s16.astype(np.float64)[..., None]
    z = z16.astype(np.float64)[..., None]
    np.testing.assert_allclose(HQ.hqq_zero_step(w, s, z, 1e30, 0.7), z, rtol=0, atol=1e-12)
    qq = np.clip(np.rint(w / s + z), 0, 7)
    np.testing.assert_allclose(HQ.hqq_zero_step(w, s, z, 1e-30, 0.7), np.mean(qq - w / s, axis=-1, keepdims=True),
                               rtol=0, atol=1e-12)


def test_zero_iterations_is_rtn():
    W = _w(32, 256, 2)
    c, s, z = HQ.quantize_hqq_int3(W, iters=0)
    q, s0, z0 = oracle.quantize_rtn_int3(W)
    np.testing.assert_array_equal(c, q)
    np.testing.assert_array_equal(s.view(np.uint16), s0.view(np.uint16))
    np.testing.assert_array_equal(z.view(np.uint16), z0.view(np.uint16))


@pytest.mark.parametrize("kind", ["normal", "heavy", "wide"])
def test_never_worse_than_rtn_and_better_on_average(kind):
    W = _w(64, 512, 3, kind)
    c, s, z = HQ.quantize_hqq_int3(W)
    q, s0, z0 = oracle.quantize_rtn_int3(W)
    np.testing.assert_array_equal(s.view(np.uint16), s0.view(np.uint16))   # scale is RTN's
    assert c.max() <= 7
    w = W.astype(np.float64).reshape(64, 8, 64)
    e_h = HQ.group_mae(w, s.astype(np.float64)[..., None], z.astype(np.float64)[..., None])
    e_r = HQ.group_mae(w, s0.astype(np.float64)[..., None], z0.astype(np.float64)[..., None])
    assert np.all(e_h <= e_r)
    assert e_h.mean() < e_r.mean()
    # the stored codes are the codes at the kept zero point
    deq = oracle.dequant_int3(c, s, z).reshape(64, 8, 64)
    np.testing.assert_allclose(np.mean(np.abs(w - deq), axis=-1), e_h, rtol=1e-12)


def test_grid_weights_stay_exact():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 8, (16, 128)).astype(np.uint8)
    codes[:, ::64] = 0
    codes[:, 1::64] = 7
    W = ((codes.astype(np.float64) - 3.0) * 0.25).astype(np.float32)
    c, s, z = HQ.quantize_hqq_int3(W)
    np.testing.assert_array_equal(c, codes)
    assert np.all(z == 3.0) and np.all(s == 0.25)


def test_threshold_active_on_unit_scale_weights():
    """With unit-scale weights the quantization errors reach the soft
    threshold's knee (|x|^(2-p) > 1/beta), so W_e is not identically zero."""
    W = _w(16, 256, 5, "wide")
    q, s16, z16 = oracle.quantize_rtn_int3(W)
    w = W.astype(np.float64).reshape(16, 4, 64)
    s = s16.astype(np.float64)[..., None]
    z = z16.astype(np.float64)[..., None]
    x = w - (np.clip(np.rint(w / s + z), 0, 7) - z) * s
    assert np.count_nonzero(HQ.shrink_lp(x, 10.0, 0.7)) > 0


def _golden_group():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hqq_cases.json")))
    w = np.zeros(64)
    w[1] = 7.0
    w[2:] = np.arange(62) % 7 + 0.25
    return g, w


def test_hqq_trajectory_hand_worked():
    """Two half-quadratic updates of one unit-scale group with p = 1/2, by
    hand (tests/golden/hqq_cases.json): the first update uses beta, the
    second beta * kappa -- a dropped or inverted schedule gives another z2."""
    g, w = _golden_group()
    q, s16, z16 = oracle.quantize_rtn_int3(w[None, :].astype(np.float32))
    assert float(s16[0, 0]) == g["group"]["rtn_scale"] and float(z16[0, 0]) == g["group"]["rtn_zero"]
    beta = g["beta_num"] / g["beta_den"]
    ws = w.reshape(1, 1, 64)
    s = np.ones((1, 1, 1))
    z0 = np.zeros((1, 1, 1))
    z2s = []
    for case in g["cases"]:
        traj = HQ.hqq_zero_trajectory(ws, s, z0, 2, g["p"], beta, case["kappa"])
        assert traj[0][0, 0, 0] == pytest.approx(g["iteration_1"]["z"], abs=1e-12)
        assert traj[1][0, 0, 0] == pytest.approx(case["z2"], abs=1e-12)
        z2s.append(case["z2"])
    assert len(set(z2s)) == len(z2s)


def test_hqq_quantizer_follows_trajectory():
    """quantize_hqq_int3 keeps the best candidate among the RTN zero point and
    f16(z_t) of the trajectory: for the hand-worked group the stored zero is
    one of those and its error is the least of them."""
    g, w = _golden_group()
    beta = g["beta_num"] / g["beta_den"]
    c, s, z = HQ.quantize_hqq_int3(w[None, :].astype(np.float32), iters=2, p=0.5, beta=beta, kappa=2.0)
    cands = [0.0, float(np.float16(-0.09)), float(np.float16(g["cases"][0]["z2"]))]
    errs = [HQ.group_mae(w.reshape(1, 1, 64), np.ones((1, 1, 1)), np.full((1, 1, 1), zc))[0, 0] for zc in cands]
    assert float(z[0, 0]) in cands
    assert HQ.group_mae(w.reshape(1, 1, 64), np.ones((1, 1, 1)), np.full((1, 1, 1), float(z[0, 0])))[0, 0] == min(errs)
