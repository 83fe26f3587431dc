"""GPU compensator construction vs the oracle (oracle/builder.py): the
randomized rank-r approximation on matrices with a spectral gap (against both
the oracle's randomized algorithm with the same test matrix and the exact
SVD), on a flat quantization-noise spectrum (energies and singular values),
and the quantize <-> compensate refinement (first iteration bit-exact codes,
later iterations within a statistical bar, fixed point on grid weights,
rank 0 = plain RTN).  Integer outputs of later rounds are checked for
validity, not by share: a round quantizes W - L with L the previous round's
factors (formed in fp32 on the GPU), so the check re-quantizes W - U V with
the GPU's own previous-round factors in float64 and allows differences only
at rounding ties (tests/int_checks.py)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import builder as OB
from tests.gpu_helpers import to_np
from tests.int_checks import assert_hqq_valid, assert_rtn_valid

pytestmark = pytest.mark.gpu


def _m():
    import extreme_quantized_moe_amd as m
    return m


def _omega(l, K, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((l, K), generator=g)


def _spectrum_matrix(N, K, sig, seed):
    rng = np.random.default_rng(seed)
    Uq, _ = np.linalg.qr(rng.standard_normal((N, len(sig))))
    Vq, _ = np.linalg.qr(rng.standard_normal((K, len(sig))))
    return ((Uq * np.asarray(sig)[None, :]) @ Vq.T).astype(np.float32)


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


@pytest.mark.parametrize("N,K,r,p,q", [(512, 256, 16, 8, 2), (2048, 512, 8, 5, 1), (300, 640, 64, 16, 2),
                                       (256, 1024, 32, 0, 3)])
def test_lowrank_svd_with_a_gap(N, K, r, p, q):
    m = _m()
    sig = np.concatenate([np.linspace(4.0, 2.0, r), np.full(min(N, K) // 2, 1e-3)])
    R = _spectrum_matrix(N, K, sig, N + K)
    om = _omega(r + p, K, r)
    U, V, s = m.lowrank_svd(torch.from_numpy(R).cuda(), r, om.cuda(), power_iters=q)
    torch.cuda.synchronize()
    L = to_np(U).astype(np.float64) @ to_np(V).astype(np.float64)
    Ue, Ve, se = OB.exact_lowrank_ref(R, r)
    Uo, Vo, so = OB.rsvd_ref(R, r, om.numpy(), q)
    np.testing.assert_allclose(to_np(s), se, rtol=2e-4)
    assert _rel(L, Ue @ Ve) <= 2e-4
    assert _rel(L, Uo @ Vo) <= 2e-4
    # balanced factors: column norms of U = row norms of V = sqrt(sigma)
    np.testing.assert_allclose(np.linalg.norm(to_np(U), axis=0), np.sqrt(se), rtol=2e-4)
    np.testing.assert_allclose(np.linalg.norm(to_np(V), axis=1), np.sqrt(se), rtol=2e-4)


def test_lowrank_svd_exact_low_rank_input():
    m = _m()
    rng = np.random.default_rng(3)
    R = (rng.standard_normal((384, 6)) @ rng.standard_normal((6, 256))).astype(np.float32)
    U, V, s = m.lowrank_svd(torch.from_numpy(R).cuda(), 8, _omega(12, 256, 4).cuda(), power_iters=1)
    torch.cuda.synchronize()
    L = to_np(U).astype(np.float64) @ to_np(V).astype(np.float64)
    assert _rel(L, R.astype(np.float64)) <= 1e-5
    # null directions: sigma is the square root of fp32 Gram noise (about
    # 1e-7 of the largest eigenvalue), their product terms stay at rounding level
    assert np.all(to_np(s)[6:] <= 2e-3 * to_np(s)[0])


def test_lowrank_svd_zero_input():
    m = _m()
    R = torch.zeros((256, 128), device="cuda")
    U, V, s = m.lowrank_svd(R, 16, _omega(24, 128, 5).cuda(), power_iters=2)
    torch.cuda.synchronize()
    assert torch.all(U == 0) and torch.all(V == 0) and torch.all(s == 0)


def _weights(N, K, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((N, K), generator=g) * 0.02


@pytest.mark.parametrize("N,K,r,p", [(512, 512, 16, 8), (1024, 256, 32, 8)])
def test_build_first_iteration(N, K, r, p):
    """iters = 1: codes are plain RTN (bit-exact); the compensator is the
    randomized rank-r approximation of the RTN residual (a flat
    quantization-noise spectrum: compared by energies and singular values)."""
    m = _m()
    W = _weights(N, K, N + r)
    om = _omega(r + p, K, 7)[None]
    codes, scale, zero, U, V, s = m.build_compensator(W.cuda(), r, 1, om.cuda(), power_iters=2)
    torch.cuda.synchronize()
    q, sc, z = oracle.quantize_rtn_int3(W.numpy())
    np.testing.assert_array_equal(to_np(codes), q)
    np.testing.assert_array_equal(to_np(scale).view(np.uint16), sc.view(np.uint16))
    np.testing.assert_array_equal(to_np(zero).view(np.uint16), z.view(np.uint16))
    R = OB.residual_ref(W.numpy(), q, sc, z)
    Uo, Vo, so = OB.rsvd_ref(R, r, om[0].numpy(), 2)
    L = to_np(U).astype(np.float64) @ to_np(V).astype(np.float64)
    np.testing.assert_allclose(to_np(s), so, rtol=2e-3)
    e_gpu, e_or = np.linalg.norm(R - L), np.linalg.norm(R - Uo @ Vo)
    assert abs(e_gpu - e_or) <= 5e-5 * e_or
    assert e_gpu < np.linalg.norm(R)


def _prev_round_residual(m, W, r, iters, om, q, quantizer="rtn"):
    """W - U V in float64 with the GPU's factors after iters rounds (the
    builder is deterministic, so these are the factors round iters + 1 of a
    longer run starts from)."""
    out = m.build_compensator(W.cuda(), r, iters, om[:iters].cuda(), power_iters=q, quantizer=quantizer)
    torch.cuda.synchronize()
    U, V = to_np(out[3]).astype(np.float64), to_np(out[4]).astype(np.float64)
    return W.numpy().astype(np.float64) - U @ V


# W - U V differs between fp32 (GPU) and float64 by a few 1e-9 at weights of
# 0.02 with scales near 0.017: w / s moves by under 1e-6 and the group extremes
# by under 1e-6 relative
_REL, _EPS = 1e-6, 1e-5


def test_build_refinement_iterations():
    """iters = 3: the final round's codes, scales and zero points are the RTN
    quantization of W - U2 V2 (the GPU's round-2 factors) except at rounding
    ties; the compensated error follows the oracle's float64 refinement with
    the same test matrices."""
    m = _m()
    N, K, r, p = 512, 512, 16, 8
    W = _weights(N, K, 11)
    om = torch.stack([_omega(r + p, K, 20 + t) for t in range(3)])
    codes, scale, zero, U, V, s = m.build_compensator(W.cuda(), r, 3, om.cuda(), power_iters=2)
    torch.cuda.synchronize()
    Wp = _prev_round_residual(m, W, r, 2, om, 2)
    nsz, nc = assert_rtn_valid(Wp, to_np(codes), to_np(scale), to_np(zero), _REL, _EPS, "round 3 of 3")
    print(f"refinement: {nsz} scale/zero groups and {nc} codes excused as rounding ties")
    ref = OB.build_ref(W.numpy(), r, 3, om.numpy(), 2)
    Wd = oracle.dequant_int3(to_np(codes), to_np(scale), to_np(zero))
    L = to_np(U).astype(np.float64) @ to_np(V).astype(np.float64)
    err = np.linalg.norm(W.numpy().astype(np.float64) - Wd - L)
    assert abs(err - ref["errors"][-1]) <= 1e-3 * ref["errors"][-1]


def test_build_fixed_point_on_grid_weights():
    m = _m()
    rng = np.random.default_rng(15)
    N, K = 128, 256
    codes = rng.integers(0, 8, (N, K)).astype(np.uint8)
    codes[:, ::64] = 0
    codes[:, 1::64] = 7
    W = torch.from_numpy(((codes.astype(np.float64) - 3.0) * 0.25).astype(np.float32))
    om = torch.stack([_omega(12, K, 30 + t) for t in range(2)])
    c, sc, z, U, V, s = m.build_compensator(W.cuda(), 8, 2, om.cuda(), power_iters=1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(c), codes)
    assert torch.all(sc == 0.25) and torch.all(z == 3.0)
    assert torch.all(U == 0) and torch.all(V == 0) and torch.all(s == 0)


def test_build_rank_zero_is_rtn():
    m = _m()
    W = _weights(256, 512, 40)
    c, sc, z, U, V, s = m.build_compensator(W.cuda(), 0, 2, None)
    torch.cuda.synchronize()
    q, s_, z_ = oracle.quantize_rtn_int3(W.numpy())
    np.testing.assert_array_equal(to_np(c), q)


def test_build_with_hqq_quantizer():
    """quantizer "hqq", 2 iterations: the first round is the HQQ-style
    quantizer on W (validated against the oracle as in the quantizer's own
    test: zero points equal except at error ties); the second is the same
    quantizer on W - U1 V1 (the GPU's round-1 factors, formed in fp32), so
    the tie and rounding-sensitivity allowances widen to the size of that
    fp32 rounding; codes are the codes at the stored zero point everywhere;
    the compensated error follows the oracle's refinement."""
    m = _m()
    N, K, r, p = 512, 512, 16, 8
    W = _weights(N, K, 50)
    om = torch.stack([_omega(r + p, K, 60 + t) for t in range(2)])
    first = m.build_compensator(W.cuda(), r, 1, om[:1].cuda(), power_iters=2, quantizer="hqq")
    out = m.build_compensator(W.cuda(), r, 2, om.cuda(), power_iters=2, quantizer="hqq")
    torch.cuda.synchronize()
    c1, s1, z1 = (to_np(t) for t in first[:3])
    assert_hqq_valid(W.numpy().astype(np.float64), c1, s1, z1, "hqq build round 1")
    codes, scale, zero, U, V, s = (to_np(t) for t in out)
    U1, V1 = to_np(first[3]).astype(np.float64), to_np(first[4]).astype(np.float64)
    Wp = W.numpy().astype(np.float64) - U1 @ V1
    nd = assert_hqq_valid(Wp, codes, scale, zero, "hqq build round 2", tie_rel=_REL, traj_rel=_REL,
                          code_eps=_EPS)
    print(f"hqq build round 2: {nd} zero points differ from the float64 run")
    ref = OB.build_ref(W.numpy(), r, 2, om.numpy(), 2, quantizer="hqq")
    Wd = oracle.dequant_int3(codes, scale, zero)
    err = np.linalg.norm(W.numpy().astype(np.float64) - Wd - U.astype(np.float64) @ V.astype(np.float64))
    assert abs(err - ref["errors"][-1]) <= 1e-3 * ref["errors"][-1]


def test_build_full_size_mixtral_matrix():
    """A Mixtral-shaped gate matrix (14336 x 4096, N(0, 0.02)) at the rank the
    benchmark uses (64, oversampling 16, 2 power iterations): RTN codes
    bit-exact, singular values and the compensated error against the oracle's
    float64 run of the same algorithm with the same test matrix."""
    m = _m()
    N, K, r, p, q = 14336, 4096, 64, 16, 2
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    W = torch.randn((N, K), generator=g, device="cuda") * 0.02
    om = torch.randn((1, r + p, K), generator=g, device="cuda")
    codes, scale, zero, U, V, s = m.build_compensator(W, r, 1, om, power_iters=q)
    torch.cuda.synchronize()
    Wh = W.cpu().numpy()
    qc, sc, z = oracle.quantize_rtn_int3(Wh)
    np.testing.assert_array_equal(to_np(codes), qc)
    R = OB.residual_ref(Wh, qc, sc, z)
    del qc, Wh
    Uo, Vo, so = OB.rsvd_ref(R, r, om[0].cpu().numpy(), q)
    np.testing.assert_allclose(to_np(s), so, rtol=2e-3)
    # ||R - L||^2 = ||R||^2 - sum sigma^2 for both (L is a projection of R)
    r2 = float(np.sum(R * R))
    e_or = r2 - float(np.sum(so.astype(np.float64) ** 2))
    e_gpu = r2 - float(np.sum(to_np(s).astype(np.float64) ** 2))
    assert abs(e_gpu - e_or) <= 1e-4 * e_or
    # and the GPU factors do form that projection: sample rows of L = U V
    rows = np.random.default_rng(1).choice(N, 256, replace=False)
    Ls = to_np(U)[rows].astype(np.float64) @ to_np(V).astype(np.float64)
    Lo = Uo[rows] @ Vo
    assert _rel(Ls, Lo) <= 5e-2          # flat spectrum: the top-64 subspace is only loosely determined
    assert abs(np.sum(Ls * Ls) - np.sum(Lo * Lo)) <= 2e-2 * np.sum(Lo * Lo)
