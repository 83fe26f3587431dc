"""GPU HQQ-style quantizer vs the oracle (oracle/hqq.py): iters = 0 is RTN
bit for bit; with the published defaults the scale is RTN's, every code is
the code at the stored zero point, and every zero point equals the oracle's
except where the two candidates' group errors tie (the GPU adds a group's
terms in another order, and a flat stretch of the l1 error decides which of
two equal candidates is kept first); no group is worse than RTN by mean
absolute error."""
import numpy as np
import pytest
import torch

import oracle
from oracle import hqq as HQ
from tests.gpu_helpers import to_np
from tests.int_checks import assert_hqq_valid

pytestmark = pytest.mark.gpu


def _m():
    import extreme_quantized_moe_amd as m
    return m


def _w(R, K, seed, kind):
    g = torch.Generator().manual_seed(seed)
    if kind == "heavy":
        torch.manual_seed(seed)
        return (torch.distributions.StudentT(3.0).sample((R, K)) * 0.02).float()
    if kind == "wide":                 # unit-scale weights: the soft threshold is active
        return torch.randn((R, K), generator=g)
    return torch.randn((R, K), generator=g) * 0.02


def test_zero_iterations_is_rtn_bit_exact():
    m = _m()
    W = _w(128, 512, 1, "normal")
    c, s, z = m.quantize_hqq_int3(W.cuda(), iters=0)
    torch.cuda.synchronize()
    q, s0, z0 = oracle.quantize_rtn_int3(W.numpy())
    np.testing.assert_array_equal(to_np(c), q)
    np.testing.assert_array_equal(to_np(s).view(np.uint16), s0.view(np.uint16))
    np.testing.assert_array_equal(to_np(z).view(np.uint16), z0.view(np.uint16))


@pytest.mark.parametrize("kind,R,K", [("normal", 256, 1024), ("heavy", 128, 1408), ("wide", 128, 512)])
def test_defaults_match_oracle(kind, R, K):
    m = _m()
    W = _w(R, K, 2, kind)
    c, s, z = m.quantize_hqq_int3(W.cuda())
    torch.cuda.synchronize()
    c, s, z = to_np(c), to_np(s), to_np(z)
    ndiff = assert_hqq_valid(W.numpy().astype(np.float64), c, s, z, f"hqq {kind} {R}x{K}")
    print(f"hqq {kind}: {ndiff} of {R * K // 64} zero points differ from the oracle, all ties")
    w = W.numpy().astype(np.float64).reshape(R, K // 64, 64)
    e_gpu = HQ.group_mae(w, s.astype(np.float64)[..., None], z.astype(np.float64)[..., None])
    q0, s0, z0 = oracle.quantize_rtn_int3(W.numpy())
    e_rtn = HQ.group_mae(w, s0.astype(np.float64)[..., None], z0.astype(np.float64)[..., None])
    assert e_gpu.mean() < 0.98 * e_rtn.mean()
