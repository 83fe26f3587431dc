"""The seeded input generators: deterministic, per-tensor seeds, shapes and
distributions of the workloads."""
import numpy as np
import torch

import synth
from synth.configs import C1, C2, C4


def test_linear_shapes_and_determinism():
    a = synth.gen_linear(C1)
    b = synth.gen_linear(C1)
    assert a["X"].shape == (16, 512) and a["X"].dtype == torch.float16
    assert a["W"].shape == (1024, 512) and a["W"].dtype == torch.float32
    assert a["A"].shape == (512, 16) and a["B"].shape == (16, 1024)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert abs(float(a["W"].std()) - 0.02) < 0.001
    assert abs(float(a["X"].float().std()) - 1.0) < 0.05


def test_per_tensor_seeds_independent():
    small = C2.with_(H=256, F=128)
    e0 = synth.gen_expert(small, 0, 0, 16)
    e1 = synth.gen_expert(small, 0, 1, 16)
    l1 = synth.gen_expert(small, 1, 0, 16)
    assert not torch.equal(e0["W1"], e1["W1"])
    assert not torch.equal(e0["W1"], l1["W1"])
    assert not torch.equal(e0["W1"], e0["W3"])
    again = synth.gen_expert(small, 0, 1, 16, which=("W3",))
    assert torch.equal(again["W3"], e1["W3"])


def test_ranks_and_zipf():
    r = synth.gen_ranks(C4)
    assert len(r) == 66 and set(r[:64]) <= {8, 16, 32} and r[64:] == [32, 32]
    lg = synth.gen_logits(C4)
    assert lg.shape == (256, 64) and lg.dtype == torch.float32
    # skew: the most popular expert is picked far more often than uniform
    top = torch.topk(lg, 6, dim=1).indices.reshape(-1)
    counts = np.bincount(top.numpy(), minlength=64)
    assert counts.max() > 4 * counts.mean()
