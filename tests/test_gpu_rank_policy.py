"""GPU inputs of the adaptive rank policy vs the oracle: per-matrix weight
kurtosis (float64 accumulation, 1e-12), routed pairs per expert accumulated
over routing calls (bit-exact), and the policy run on them."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import to_np

pytestmark = pytest.mark.gpu


def _m():
    import extreme_quantized_moe_amd as m
    return m


def test_kurtosis_matches_oracle():
    m = _m()
    g = torch.Generator().manual_seed(1)
    mats = [torch.randn((96, 256), generator=g) * 0.02,                    # Gaussian: about 3
            (torch.rand((96, 256), generator=g) * 2 - 1) * 0.05,           # uniform: about 1.8
            torch.distributions.StudentT(4.0).sample((96, 256)) * 0.02,    # heavy tails
            torch.full((96, 256), 0.5),                                    # constant: 0
            torch.randn((96, 256), generator=g) * 0.02 + 3.0]              # offset mean
    W = torch.stack([x.float() for x in mats])
    kurt, mean = m.weight_kurtosis(W.cuda())
    torch.cuda.synchronize()
    for i, x in enumerate(mats):
        want = oracle.kurtosis_ref(x.numpy())
        assert float(kurt[i]) == pytest.approx(want, rel=1e-12, abs=1e-300), i
        assert float(mean[i]) == pytest.approx(float(np.mean(x.numpy().astype(np.float64))), rel=1e-12, abs=1e-15)


def test_kurtosis_large_and_odd_sizes():
    m = _m()
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    W = torch.randn((3, 4096 * 1412), generator=g, device="cuda")   # not a multiple of the block chunk
    W[1] = W[1] ** 3
    kurt, _ = m.weight_kurtosis(W, count=3)
    torch.cuda.synchronize()
    Wh = W.cpu().numpy()
    for i in range(3):
        assert float(kurt[i]) == pytest.approx(oracle.kurtosis_ref(Wh[i]), rel=1e-11)


def test_expert_counts_and_policy():
    m = _m()
    T, E, k, S = 512, 8, 2, 1
    counts = torch.zeros(E + S, dtype=torch.int64, device="cuda")
    want = np.zeros(E + S, dtype=np.int64)
    for b in range(4):
        g = torch.Generator().manual_seed(10 + b)
        logits = torch.randn((T, E), generator=g)
        logits[:, 3] += 1.0                       # one popular expert
        r = m.route_sort(logits.cuda(), k, S, True)
        m.expert_counts(r["offsets"], counts)
        off = oracle.route_ref(logits.numpy(), k, S, True)["offsets"]
        want += np.diff(off)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(counts), want)
    freq = to_np(counts) / (4.0 * T)
    assert freq[-1] == 1.0
    kurt = [3.0 + 0.1 * e for e in range(E + S)]
    dense = [False] * E + [True]
    ranks = m.rank_policy(kurt, list(freq), dense, 8 * 32)
    assert ranks == oracle.rank_policy_ref(kurt, list(freq), dense, 8 * 32)
    assert ranks[-1] == max(ranks)                # the shared expert
    assert ranks[3] == max(ranks[:E])             # the popular routed expert
