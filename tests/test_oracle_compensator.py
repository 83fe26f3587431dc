"""Pins for the oracle's int3 compensators (oracle/compensator.py): a
hand-worked quantization of one U row, the weights' golden g64 cases placed in
a V row, the RTN error bound on both factors, the group axes, hand-derived
packed words of both layouts, a second packer that walks the spec one code at
a time, round trips, and the bound the factor rounding puts on the
compensated product."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import compensator as OC

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CASES = json.load(open(os.path.join(GOLD, "compensator_cases.json")))
QCASES = json.load(open(os.path.join(GOLD, "quant_cases.json")))["cases"]


def _factors(K, N, r, seed, sigma=0.01):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((K, r)) * sigma).astype(np.float16)
    B = (rng.standard_normal((r, N)) * sigma).astype(np.float16)
    return A, B


def test_golden_u_row():
    c = CASES["u_row"]
    A, B = _factors(128, 64, 8, 1)
    B[:, 5] = np.array(c["values"], dtype=np.float16)      # U row n = 5
    q = OC.quantize_compensator(A, B)
    np.testing.assert_array_equal(q["u_codes"][5], c["codes"])
    assert int(oracle.f16_bits(q["u_scale"][5, 0])) == c["scale_bits"]
    assert int(oracle.f16_bits(q["u_zero"][5, 0])) == c["zero_bits"]


@pytest.mark.parametrize("case", QCASES, ids=lambda c: c["name"])
def test_golden_g64_cases_in_a_v_row(case):
    """V = A^T is grouped like the weights: 64 consecutive k of one rank row."""
    vals = list(case["values_head"]) + [case["fill"]] * (64 - len(case["values_head"]))
    codes = list(case["codes_head"]) + [case["code_fill"]] * (64 - len(case["codes_head"]))
    if not np.all(np.asarray(vals, np.float16).astype(np.float64) == np.asarray(vals, np.float64)):
        pytest.skip("case values are not float16-exact (factors are float16)")
    A, B = _factors(256, 64, 16, 2)
    A[64:128, 3] = np.asarray(vals, dtype=np.float16)      # rank row j = 3, group 1
    q = OC.quantize_compensator(A, B)
    np.testing.assert_array_equal(q["v_codes"][3, 64:128], codes)


@pytest.mark.parametrize("r", [8, 16, 24, 32, 64])
def test_rtn_bound_and_extremes(r):
    K, N = 256, 128
    A, B = _factors(K, N, r, r)
    q = OC.quantize_compensator(A, B)
    Ad, Bd = OC.dequant_compensator(q)
    vs = np.repeat(q["v_scale"].astype(np.float64), 64, axis=1).T   # [K][r]
    us = q["u_scale"].astype(np.float64).T                          # [1][N] over all r
    tol = 1e-12
    assert np.all(np.abs(A.astype(np.float64) - Ad) <= vs / 2 * (1 + tol))
    assert np.all(np.abs(B.astype(np.float64) - Bd) <= us / 2 * (1 + tol))
    for codes in (q["v_codes"].reshape(r, K // 64, 64), q["u_codes"][:, None, :]):
        assert codes.max() <= 7
        assert np.all(codes.min(axis=2) == 0) and np.all(codes.max(axis=2) == 7)


def test_group_axes():
    """Changing one U entry changes only its own row's scale/zero (one group per
    output row, over the ranks); changing one A entry changes only its rank
    row's 64-wide group."""
    A, B = _factors(256, 64, 16, 3)
    q0 = OC.quantize_compensator(A, B)
    B2 = B.copy()
    B2[4, 10] = np.float16(0.5)                              # U[10][4]
    q1 = OC.quantize_compensator(A, B2)
    changed = np.nonzero(q0["u_scale"][:, 0] != q1["u_scale"][:, 0])[0]
    assert list(changed) == [10]
    A2 = A.copy()
    A2[130, 7] = np.float16(0.5)                             # V[7][130], group 2
    q2 = OC.quantize_compensator(A2, B)
    diff = np.argwhere(q0["v_scale"] != q2["v_scale"])
    assert diff.tolist() == [[7, 2]]


def test_rank_zero():
    A = np.zeros((128, 0), np.float16)
    B = np.zeros((0, 64), np.float16)
    q = OC.quantize_compensator(A, B)
    Ad, Bd = OC.dequant_compensator(q)
    assert Ad.shape == (128, 0) and Bd.shape == (0, 64)
    words, sz = OC.pack_lr_v(q["v_codes"], q["v_scale"], q["v_zero"], 16)
    assert not words.any() and np.all(sz == OC.PAD_SZ_WORD)


def test_product_within_rounding_bound():
    """(X A_d) B_d differs from (X A) B by at most |X| |A - A_d| |B| +
    |X A_d| |B - B_d| (elementwise), with |A - A_d| <= s/2 from the RTN rule:
    a dropped zero point or a wrong group scale breaks it."""
    K, N, r, M = 512, 256, 32, 8
    A, B = _factors(K, N, r, 4)
    X = np.random.default_rng(5).standard_normal((M, K)).astype(np.float16).astype(np.float64)
    q = OC.quantize_compensator(A, B)
    Ad, Bd = OC.dequant_compensator(q)
    Af, Bf = A.astype(np.float64), B.astype(np.float64)
    got = (X @ Ad) @ Bd
    exact = (X @ Af) @ Bf
    dA = np.repeat(q["v_scale"].astype(np.float64), 64, axis=1).T / 2
    dB = np.broadcast_to(q["u_scale"].astype(np.float64).T / 2, Bf.shape)
    bound = np.abs(X) @ dA @ np.abs(Bf) + np.abs(X @ Ad) @ dB
    assert np.all(np.abs(got - exact) <= bound * (1 + 1e-9))
    # the int3 rounding of random Gaussian factors is a sizeable but bounded part of the term
    assert np.linalg.norm(got - exact) < 0.5 * np.linalg.norm(exact)


@pytest.mark.parametrize("case", CASES["v_layout"], ids=lambda c: c["why"][:30])
def test_golden_v_words(case):
    R, K = case["max_rank"], case["K"]
    codes = np.zeros((R, K), np.uint8)
    for j, k, v in case["set"]:
        codes[j, k] = v
    s = np.ones((R, K // 64), np.float16)
    z = np.zeros((R, K // 64), np.float16)
    words, _ = OC.pack_lr_v(codes, s, z, R)
    nz = {int(i): int(words[i]) for i in np.nonzero(words)[0]}
    assert nz == {int(i): v for i, v in case["expect"].items()}
    scal = OC.pack_lr_v_scalar(codes.tolist(), R)
    assert {i: v for i, v in enumerate(scal) if v} == nz


@pytest.mark.parametrize("case", CASES["u_layout"], ids=lambda c: c["why"][:30])
def test_golden_u_words(case):
    N, R = case["N"], case["max_rank"]
    codes = np.zeros((N, R), np.uint8)
    for n, j, v in case["set"]:
        codes[n, j] = v
    words, _ = OC.pack_lr_u(codes, np.ones(N, np.float16), np.zeros(N, np.float16), R)
    nz = {int(i): int(words[i]) for i in np.nonzero(words)[0]}
    assert nz == {int(i): v for i, v in case["expect"].items()}
    scal = OC.pack_lr_u_scalar(codes.tolist(), R)
    assert {i: v for i, v in enumerate(scal) if v} == nz


@pytest.mark.parametrize("case", CASES["v_sz"], ids=str)
def test_golden_v_sz(case):
    R, K = case["max_rank"], case["K"]
    s = np.zeros((R, K // 64), np.float16)
    z = np.zeros((R, K // 64), np.float16)
    s[case["j"], case["gg"]] = np.float16(0.25)            # 0x3400
    z[case["j"], case["gg"]] = np.float16(3.5)             # 0x4300
    _, sz = OC.pack_lr_v(np.zeros((R, K), np.uint8), s, z, R)
    assert int(sz[case["word"]]) == 0x43003400
    assert int(np.sum(sz == 0x43003400)) == 1


@pytest.mark.parametrize("case", CASES["u_sz"], ids=str)
def test_golden_u_sz(case):
    N = case["N"]
    s = np.zeros(N, np.float16)
    z = np.zeros(N, np.float16)
    s[case["n"]] = np.float16(0.25)
    z[case["n"]] = np.float16(3.5)
    _, sz = OC.pack_lr_u(np.zeros((N, 8), np.uint8), s, z, 8)
    assert int(sz[case["word"]]) == 0x43003400
    assert int(np.sum(sz == 0x43003400)) == 1


@pytest.mark.parametrize("rank,max_rank,K", [(16, 16, 128), (8, 16, 256), (24, 32, 384), (64, 64, 128), (40, 64, 256)])
def test_v_round_trip_and_scalar(rank, max_rank, K):
    rng = np.random.default_rng(rank * 7 + K)
    codes = rng.integers(0, 8, (rank, K), dtype=np.uint8)
    s = (rng.uniform(0.001, 0.01, (rank, K // 64))).astype(np.float16)
    z = (rng.uniform(0, 7, (rank, K // 64))).astype(np.float16)
    words, sz = OC.pack_lr_v(codes, s, z, max_rank)
    assert words.size == OC.lr_v_words(max_rank, K) and words.size * 32 == 3 * max_rank * K
    assert sz.size == OC.lr_v_sz_words(max_rank, K)
    scal = np.array(OC.pack_lr_v_scalar(codes.tolist(), max_rank), dtype=np.uint32)
    np.testing.assert_array_equal(words, scal)
    c2, s2, z2 = OC.unpack_lr_v(words, sz, max_rank, K)
    np.testing.assert_array_equal(c2[:rank], codes)
    assert not c2[rank:].any()
    np.testing.assert_array_equal(s2[:rank], s)
    np.testing.assert_array_equal(z2[:rank], z)
    assert np.all(s2[rank:] == 1) and np.all(z2[rank:] == 0)


@pytest.mark.parametrize("N,rank,max_rank", [(64, 8, 8), (128, 16, 32), (64, 24, 32), (192, 64, 64), (64, 40, 64)])
def test_u_round_trip_and_scalar(N, rank, max_rank):
    rng = np.random.default_rng(N + rank)
    codes = rng.integers(0, 8, (N, rank), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, N).astype(np.float16)
    z = rng.uniform(0, 7, N).astype(np.float16)
    words, sz = OC.pack_lr_u(codes, s, z, max_rank)
    assert words.size == OC.lr_u_words(N, max_rank) and sz.size == N
    scal = np.array(OC.pack_lr_u_scalar(codes.tolist(), max_rank), dtype=np.uint32)
    np.testing.assert_array_equal(words, scal)
    c2, s2, z2 = OC.unpack_lr_u(words, sz, N, max_rank)
    np.testing.assert_array_equal(c2[:, :rank], codes)
    assert not c2[:, rank:].any()
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(z2, z)


def test_every_bit_used_once():
    """All 96 bits of a triplet carry a code: all-sevens fills every word."""
    words, _ = OC.pack_lr_v(np.full((16, 128), 7, np.uint8), np.ones((16, 2), np.float16),
                            np.zeros((16, 2), np.float16), 16)
    # bits 0 and 16 of planes hold pair 15; bits 1..15 and 17..31 the rest
    assert np.all(words == 0xFFFFFFFF)
    words, _ = OC.pack_lr_u(np.full((64, 32), 7, np.uint8), np.ones(64, np.float16),
                            np.zeros(64, np.float16), 32)
    assert np.all(words == 0xFFFFFFFF)


def test_quantize_expert_int3_uses_the_dequantized_factors():
    rng = np.random.default_rng(9)
    exp = {"W1": (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)}
    exp["A1"], exp["B1"] = _factors(128, 64, 16, 10)
    fp = oracle.quantize_expert(exp)
    q3 = oracle.quantize_expert(exp, lr_format="int3")
    np.testing.assert_array_equal(fp["W1"][0], q3["W1"][0])
    Ad, Bd = OC.dequant_compensator(OC.quantize_compensator(exp["A1"], exp["B1"]))
    np.testing.assert_array_equal(q3["A1"], Ad)
    np.testing.assert_array_equal(q3["B1"], Bd)
    assert not np.array_equal(q3["A1"], fp["A1"].astype(np.float64))
