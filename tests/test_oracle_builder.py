"""Pins for the oracle's compensator construction (oracle/builder.py): the
Eckart-Young facts of the truncated SVD, exact recovery of matrices of rank at
most r by the randomized subspace iteration, agreement with the exact SVD
where the spectrum has a gap, the lower bound every rank-r approximation
obeys, and the structure of the refinement loop (first iteration = plain
RTN, the SVD step never increases the error, rank 0 = no compensator)."""
import numpy as np
import pytest

import oracle
from oracle import builder as OB


def _omega(l, K, seed):
    return np.random.default_rng(seed).standard_normal((l, K))


def _spectrum_matrix(N, K, sig, seed):
    """N x K with singular values sig (len <= min(N, K)) and random singular
    vectors."""
    rng = np.random.default_rng(seed)
    Uq, _ = np.linalg.qr(rng.standard_normal((N, len(sig))))
    Vq, _ = np.linalg.qr(rng.standard_normal((K, len(sig))))
    return (Uq * np.asarray(sig)[None, :]) @ Vq.T


@pytest.mark.parametrize("r", [1, 8, 16])
def test_eckart_young_tail_energy(r):
    R = np.random.default_rng(r).standard_normal((96, 64))
    U, V, s = OB.exact_lowrank_ref(R, r)
    full = np.linalg.svd(R, compute_uv=False)
    err2 = np.linalg.norm(R - U @ V) ** 2
    assert err2 == pytest.approx(np.sum(full[r:] ** 2), rel=1e-10)
    np.testing.assert_allclose(s, full[:r], rtol=1e-12)
    # balanced split: column norms of U equal row norms of V (= sqrt sigma)
    np.testing.assert_allclose(np.linalg.norm(U, axis=0), np.sqrt(s), rtol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(V, axis=1), np.sqrt(s), rtol=1e-10)


@pytest.mark.parametrize("rank_true,r,p", [(4, 8, 4), (8, 8, 0), (16, 16, 8)])
def test_rsvd_recovers_low_rank_exactly(rank_true, r, p):
    """A matrix of rank <= r is reproduced exactly for any test matrix."""
    rng = np.random.default_rng(rank_true)
    R = rng.standard_normal((200, rank_true)) @ rng.standard_normal((rank_true, 128))
    U, V, s = OB.rsvd_ref(R, r, _omega(r + p, 128, 1), power_iters=0)
    assert np.linalg.norm(R - U @ V) <= 1e-10 * np.linalg.norm(R)


@pytest.mark.parametrize("q", [0, 1, 2])
def test_rsvd_matches_exact_svd_with_a_gap(q):
    sig = np.concatenate([np.linspace(10, 5, 16), np.full(48, 1e-3)])
    R = _spectrum_matrix(256, 128, sig, 3)
    Ue, Ve, se = OB.exact_lowrank_ref(R, 16)
    Ur, Vr, sr = OB.rsvd_ref(R, 16, _omega(24, 128, 4), power_iters=q)
    # without power iterations the tail leaks in at about sigma_17 / sigma_16
    # (1e-3 / 5); every power iteration multiplies that by the squared ratio
    tol = {0: 2e-3, 1: 1e-7, 2: 1e-9}[q]
    np.testing.assert_allclose(sr, se, rtol=tol)
    assert np.linalg.norm(Ur @ Vr - Ue @ Ve) <= tol * np.linalg.norm(Ue @ Ve)


def test_any_rank_r_approximation_obeys_the_tail_bound():
    R = np.random.default_rng(5).standard_normal((128, 128))    # flat spectrum
    full = np.linalg.svd(R, compute_uv=False)
    for q in (0, 2):
        U, V, s = OB.rsvd_ref(R, 16, _omega(24, 128, 6 + q), power_iters=q)
        err2 = np.linalg.norm(R - U @ V) ** 2
        assert err2 >= np.sum(full[16:] ** 2) * (1 - 1e-12)
        # and it captures a real share of the top energy
        assert np.linalg.norm(U @ V) ** 2 >= 0.5 * np.sum(full[:16] ** 2)


def test_power_iterations_do_not_hurt_on_a_decaying_spectrum():
    sig = 1.0 / (1.0 + np.arange(96)) ** 1.5
    R = _spectrum_matrix(192, 96, sig, 7)
    tail = np.sum(sig[8:] ** 2)
    errs = []
    for q in (0, 1, 3):
        U, V, _ = OB.rsvd_ref(R, 8, _omega(12, 96, 8), power_iters=q)
        errs.append(np.linalg.norm(R - U @ V) ** 2)
    assert errs[2] <= errs[0] * (1 + 1e-9)
    assert errs[2] <= tail * 1.01


def test_residual_is_weight_minus_dequant():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    q, s, z = oracle.quantize_rtn_int3(W)
    R = OB.residual_ref(W, q, s, z)
    assert np.all(np.abs(R) <= np.repeat(s.astype(np.float64), 64, axis=1) / 2 * (1 + 1e-12))
    np.testing.assert_array_equal(R + oracle.dequant_int3(q, s, z), W.astype(np.float64))


def _weights(N, K, seed):
    return (np.random.default_rng(seed).standard_normal((N, K)) * 0.02).astype(np.float32)


def test_build_first_iteration_is_rtn_plus_svd_of_its_residual():
    W = _weights(128, 256, 10)
    om = np.stack([_omega(20, 256, 11)])
    out = OB.build_ref(W, 16, 1, om, power_iters=2)
    q, s, z = oracle.quantize_rtn_int3(W)
    np.testing.assert_array_equal(out["codes"], q)
    U, V, sg = OB.rsvd_ref(OB.residual_ref(W, q, s, z), 16, om[0], 2)
    np.testing.assert_allclose(out["U"] @ out["V"], U @ V, rtol=0, atol=1e-15)


def test_build_svd_step_never_increases_the_error():
    W = _weights(128, 256, 12)
    om = np.stack([_omega(24, 256, 13 + t) for t in range(3)])
    out = OB.build_ref(W, 16, 3, om, power_iters=2)
    for e, rn in zip(out["errors"], out["residual_norms"]):
        assert e <= rn
    # the compensated error stays well below the plain RTN error
    assert out["errors"][-1] < out["residual_norms"][0]


def test_build_rank_zero_is_plain_rtn():
    W = _weights(64, 128, 14)
    out = OB.build_ref(W, 0, 2, np.zeros((2, 0, 128)), power_iters=1)
    q, s, z = oracle.quantize_rtn_int3(W)
    np.testing.assert_array_equal(out["codes"], q)
    assert out["U"].shape == (64, 0) and out["errors"][-1] == pytest.approx(out["residual_norms"][-1])


def test_build_fixed_point_on_grid_weights():
    """Weights that lie on their own RTN grid (every group holds codes 0 and 7,
    scale 0.25, zero 3 exactly) quantize without error: the residual is zero,
    the compensator is zero, and every iteration returns the same codes."""
    rng = np.random.default_rng(15)
    N, K = 64, 128
    codes = rng.integers(0, 8, (N, K)).astype(np.uint8)
    codes[:, ::64] = 0
    codes[:, 1::64] = 7
    W = ((codes.astype(np.float64) - 3.0) * 0.25).astype(np.float32)
    om = np.stack([_omega(12, K, 17 + t) for t in range(3)])
    out = OB.build_ref(W, 8, 3, om, power_iters=1)
    np.testing.assert_array_equal(out["codes"], codes)
    assert np.all(out["scale"] == 0.25) and np.all(out["zero"] == 3.0)
    assert max(out["residual_norms"]) == 0.0 and max(out["errors"]) == 0.0
    assert np.all(out["sigma"] == 0.0)


def test_build_with_hqq_quantizer():
    """quantizer "hqq": the first iteration quantizes W with the HQQ-style
    quantizer of oracle/hqq.py and compensates its residual; grid weights are
    still a fixed point; the compensated error stays below HQQ's own error."""
    W = _weights(128, 256, 16)
    om = np.stack([_omega(24, 256, 17 + t) for t in range(2)])
    one = OB.build_ref(W, 16, 1, om[:1], power_iters=2, quantizer="hqq")
    from oracle import hqq as HQ
    q, s, z = HQ.quantize_hqq_int3(W)
    np.testing.assert_array_equal(one["codes"], q)
    np.testing.assert_array_equal(one["zero"].view(np.uint16), z.view(np.uint16))
    U, V, sg = OB.rsvd_ref(OB.residual_ref(W, q, s, z), 16, om[0], 2)
    np.testing.assert_allclose(one["U"] @ one["V"], U @ V, rtol=0, atol=1e-15)
    two = OB.build_ref(W, 16, 2, om, power_iters=2, quantizer="hqq")
    assert two["errors"][-1] < two["residual_norms"][0]
    rng = np.random.default_rng(18)
    codes = rng.integers(0, 8, (64, 128)).astype(np.uint8)
    codes[:, ::64] = 0
    codes[:, 1::64] = 7
    G = ((codes.astype(np.float64) - 3.0) * 0.25).astype(np.float32)
    out = OB.build_ref(G, 8, 2, np.stack([_omega(12, 128, 19 + t) for t in range(2)]), 1, quantizer="hqq")
    np.testing.assert_array_equal(out["codes"], codes)
    assert max(out["errors"]) == 0.0
