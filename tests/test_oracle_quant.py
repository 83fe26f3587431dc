"""Pins for the oracle's RTN int3 quantizer (oracle/quant.py) against
hand-worked cases, textbook float16 facts and properties that hold for any
correct round-to-nearest asymmetric quantizer."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _group(case):
    vals = list(case["values_head"]) + [case["fill"]] * (64 - len(case["values_head"]))
    codes = list(case["codes_head"]) + [case["code_fill"]] * (64 - len(case["codes_head"]))
    return np.array(vals, dtype=np.float32)[None, :], np.array(codes, dtype=np.uint8)[None, :]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "quant_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_golden_quant(case):
    W, codes = _group(case)
    q, s, z = oracle.quantize_rtn_int3(W)
    np.testing.assert_array_equal(q, codes)
    if "scale_bits" in case:
        assert int(oracle.f16_bits(s)[0, 0]) == case["scale_bits"]
        assert int(oracle.f16_bits(z)[0, 0]) == case["zero_bits"]
    else:
        assert float(s[0, 0]) == case["scale"]
        assert float(z[0, 0]) == case["zero"]


def test_f16_rounding_textbook():
    # IEEE binary16 facts: max finite 65504; 65519 rounds down, 65520 overflows;
    # ties go to even; 0.1 -> 0x2E66; smallest subnormal 2^-24.
    assert float(oracle.f16_rne(65519.0)) == 65504.0
    assert np.isinf(oracle.f16_rne(65520.0))
    assert float(oracle.f16_rne(1 + 2.0 ** -11)) == 1.0
    assert float(oracle.f16_rne(1 + 3 * 2.0 ** -11)) == 1 + 2.0 ** -9
    assert int(oracle.f16_bits(oracle.f16_rne(0.1))) == 0x2E66
    assert float(oracle.f16_rne(2.0 ** -24)) == 2.0 ** -24
    # direct double rounding would differ from going through float32 here:
    x = 1 + 2.0 ** -11 + 2.0 ** -40   # just above a tie -> rounds up
    assert float(oracle.f16_rne(x)) == 1 + 2.0 ** -10


def _weights(kind, R, K, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
    if kind == "heavy":
        return (rng.standard_t(3, (R, K)) * 0.02).astype(np.float32)
    return rng.uniform(-1, 1, (R, K)).astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "heavy", "uniform"])
def test_error_bound_half_scale(kind):
    W = _weights(kind, 96, 256, 1)
    q, s, z = oracle.quantize_rtn_int3(W)
    deq = oracle.dequant_int3(q, s, z)
    sb = np.repeat(s.astype(np.float64), 64, axis=1)
    err = np.abs(W.astype(np.float64) - deq)
    assert np.all(err <= sb / 2 * (1 + 1e-12))
    assert q.max() <= 7


@pytest.mark.parametrize("kind", ["normal", "heavy", "uniform"])
def test_extremes_map_to_end_codes(kind):
    W = _weights(kind, 64, 128, 2)
    q, s, z = oracle.quantize_rtn_int3(W)
    Wg = W.reshape(64, 2, 64)
    qg = q.reshape(64, 2, 64)
    imin = Wg.argmin(axis=2)
    imax = Wg.argmax(axis=2)
    assert np.all(np.take_along_axis(qg, imin[..., None], 2) == 0)
    assert np.all(np.take_along_axis(qg, imax[..., None], 2) == 7)


def test_requantize_dequantized_is_identity():
    W = _weights("normal", 64, 256, 3)
    q, s, z = oracle.quantize_rtn_int3(W)
    deq = oracle.dequant_int3(q, s, z)
    sg = np.repeat(s.astype(np.float64), 64, axis=1)
    zg = np.repeat(z.astype(np.float64), 64, axis=1)
    q2 = np.clip(np.rint(deq / sg + zg), 0, 7)
    np.testing.assert_array_equal(q2, q)


def test_code_is_nearest_level_brute_force():
    # independent of the rint formula: search all 8 levels (q - z) s
    W = _weights("uniform", 8, 128, 4)
    q, s, z = oracle.quantize_rtn_int3(W)
    sg = np.repeat(s.astype(np.float64), 64, axis=1)
    zg = np.repeat(z.astype(np.float64), 64, axis=1)
    levels = (np.arange(8)[None, None, :] - zg[..., None]) * sg[..., None]
    d = np.abs(W.astype(np.float64)[..., None] - levels)
    best = d.argmin(axis=2)
    dmin = d.min(axis=2)
    dq = np.take_along_axis(d, q[..., None].astype(np.int64), 2)[..., 0]
    # equal distance (a tie) is the only way the two may disagree
    assert np.all((best == q) | np.isclose(dq, dmin, rtol=0, atol=1e-15))


def test_group_independence():
    # changing one group must not change codes of any other group
    W = _weights("normal", 64, 256, 5)
    q, s, z = oracle.quantize_rtn_int3(W)
    W2 = W.copy()
    W2[:, 64:128] *= 10
    q2, s2, z2 = oracle.quantize_rtn_int3(W2)
    keep = np.r_[0:64, 128:256]
    np.testing.assert_array_equal(q[:, keep], q2[:, keep])
    np.testing.assert_array_equal(s[:, [0, 2, 3]], s2[:, [0, 2, 3]])
