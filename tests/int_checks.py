"""Validity checks for integer outputs whose float64 decision may
legitimately differ between the GPU and the oracle (test infrastructure).

The library and the oracle take every quantization decision in float64 with
the same operations, but some inputs reach the decision through arithmetic
in another order or precision (a compensated residual W - U V formed in fp32
on the GPU, the sums of a zero-point update added in a lane tree).  Where the
two sides differ, these helpers require that the difference is one that
rounding order can cause -- a value within a stated distance of a rounding
boundary, or two candidates whose objective values tie -- and that every
other output is bit-exact.  Nothing is compared by share."""
import numpy as np

import oracle
from oracle import hqq as HQ


def near_f16_midpoint(x, rel):
    """True where float64 x lies within rel * |x| of the midpoint between two
    neighbouring float16 values (so a perturbation of that size can flip its
    float16 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    d = rel * np.abs(x) + 1e-300
    return oracle.f16_rne(x - d).view(np.uint16) != oracle.f16_rne(x + d).view(np.uint16)


def code_ties(w, s, z, eps):
    """True where w / s + z lies within eps of a half-integer (a rounding tie
    of the code decision)."""
    t = np.asarray(w, np.float64) / s + z
    return np.abs(t - np.floor(t) - 0.5) < eps


def _codes_at(w, s, z):
    return np.clip(np.rint(w / s + z), 0.0, 7.0)


def assert_codes_consistent(W, codes, scale, zero, eps, what, group=64):
    """codes == clip(rint(w / s + z), 0, 7) with the output's own s and z,
    except at weights within eps of a rounding tie.  Returns the number of
    tie-excused differences."""
    R, K = W.shape
    w = np.asarray(W, np.float64).reshape(R, K // group, group)
    s = np.asarray(scale, np.float64)[..., None]
    z = np.asarray(zero, np.float64)[..., None]
    c = np.asarray(codes).reshape(R, K // group, group).astype(np.float64)
    bad = c != _codes_at(w, s, z)
    excused = bad & code_ties(w, s, z, eps)
    assert np.array_equal(bad, excused), (
        f"{what}: {int(np.count_nonzero(bad & ~excused))} codes differ from rint(w/s + z) away from a tie")
    return int(np.count_nonzero(excused))


def assert_rtn_valid(W, codes, scale, zero, rel, eps, what):
    """The output (codes, scale, zero) is the RTN int3 g64 quantization of
    the float64 matrix W, up to rounding-order effects of size rel on the
    group extremes: scale and zero bit-exact except in groups whose unrounded
    (hi - lo) / 7 or -lo / s lies near a float16 midpoint; codes bit-exact
    for the output's own scale and zero except at ties.  Returns
    (excused scale/zero groups, excused codes)."""
    W = np.asarray(W, np.float64)
    R, K = W.shape
    q, s_o, z_o = oracle.quantize_rtn_int3(W)
    s, z = np.asarray(scale), np.asarray(zero)
    wg = W.reshape(R, K // 64, 64)
    lo, hi = wg.min(axis=2), wg.max(axis=2)
    ds = s.view(np.uint16) != s_o.view(np.uint16)
    ok_s = ~ds | near_f16_midpoint((hi - lo) / 7.0, rel)
    assert np.all(ok_s), f"{what}: {int(np.count_nonzero(~ok_s))} scales differ away from an fp16 midpoint"
    dz = (z.view(np.uint16) != z_o.view(np.uint16)) & ~ds
    s64 = s.astype(np.float64)
    ok_z = ~dz | near_f16_midpoint(-lo / s64, rel)
    assert np.all(ok_z), f"{what}: {int(np.count_nonzero(~ok_z))} zero points differ away from an fp16 midpoint"
    n_codes = assert_codes_consistent(W, codes, s, z, eps, what)
    return int(np.count_nonzero(ds | dz)), n_codes


def assert_hqq_valid(W, codes, scale, zero, what, iters=20, p=0.7, beta=10.0, kappa=1.01,
                     tie_rel=1e-12, traj_rel=1e-12, code_eps=1e-12):
    """The output is the HQQ-style quantization of the float64 matrix W
    (oracle/hqq.py) up to rounding order of size traj_rel / code_eps:
      * the scale is the RTN scale, bit-exact except in groups whose unrounded
        (hi - lo) / 7 lies near a float16 midpoint (those groups are
        excused from the zero-point check);
      * codes are bit-exact for the output's own scale and zero point except
        at ties within code_eps;
      * where the zero point differs from the oracle's, either the two
        candidates' group errors tie (within tie_rel, relative), or the
        oracle's trajectory is rounding-sensitive in that group: its start
        -lo / s or an iterate z_t within traj_rel of a float16 midpoint (its
        candidate can round the other way), or a weight within code_eps of a
        code tie at some z_t (the update's codes can differ);
      * no group's error exceeds the RTN error.
    Returns the number of groups whose zero point differs."""
    W = np.asarray(W, np.float64)
    R, K = W.shape
    _, s_rtn, z_rtn = oracle.quantize_rtn_int3(W)
    w = W.reshape(R, K // 64, 64)
    s = np.asarray(scale)
    ds = s.view(np.uint16) != s_rtn.view(np.uint16)
    lo, hi = w.min(axis=2), w.max(axis=2)
    ok_s = ~ds | near_f16_midpoint((hi - lo) / 7.0, traj_rel)
    assert np.all(ok_s), f"{what}: {int(np.count_nonzero(~ok_s))} scales differ from RTN away from an fp16 midpoint"
    z = np.asarray(zero)
    assert_codes_consistent(W, codes, s, z, code_eps, what)
    _, _, z_o = HQ.quantize_hqq_int3(W, iters=iters, p=p, beta=beta, kappa=kappa)
    s3 = s_rtn.astype(np.float64)[..., None]
    e_gpu = HQ.group_mae(w, s3, z.astype(np.float64)[..., None])
    e_or = HQ.group_mae(w, s3, z_o.astype(np.float64)[..., None])
    e_rtn = HQ.group_mae(w, s3, z_rtn.astype(np.float64)[..., None])
    worse = (e_gpu > e_rtn * (1 + 1e-12)) & ~ds
    assert not np.any(worse), f"{what}: {int(np.count_nonzero(worse))} groups worse than RTN"
    dz = (z.view(np.uint16) != z_o.view(np.uint16)) & ~ds
    if not np.any(dz):
        return 0
    tie = np.abs(e_gpu - e_or) <= tie_rel * e_or
    sensitive = np.zeros_like(dz)
    z_t = z_rtn.astype(np.float64)[..., None]
    for zt in HQ.hqq_zero_trajectory(w, s3, z_t, iters, p, beta, kappa):
        sensitive |= near_f16_midpoint(zt[..., 0], traj_rel)
        sensitive |= np.any(code_ties(w, s3, zt, code_eps), axis=-1)
    sensitive |= np.any(code_ties(w, s3, z_t, code_eps), axis=-1)
    # the starting point itself: the RTN zero point f16(-lo / s)
    sensitive |= near_f16_midpoint(-lo / s3[..., 0], traj_rel)
    ok = ~dz | tie | sensitive
    if not np.all(ok):
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(
            f"{what}: {int(np.count_nonzero(~ok))} of {int(np.count_nonzero(dz))} differing zero points neither "
            f"tie nor follow a rounding-sensitive trajectory; first: group ({i}, {j}) z {float(z[i, j])} vs "
            f"{float(z_o[i, j])}, error {e_gpu[i, j]:.17g} vs {e_or[i, j]:.17g} (RTN {e_rtn[i, j]:.17g}), "
            f"RTN zero {float(z_rtn[i, j])}, -lo/s {float(-lo[i, j] / s3[i, j, 0]):.17g}")
    return int(np.count_nonzero(dz))
