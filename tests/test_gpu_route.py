"""GPU router vs the oracle: ids, sorted pairs, positions and offsets
bit-exact; weights to 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import C2, C3, C4
from tests.gpu_helpers import to_np

pytestmark = pytest.mark.gpu


def _check(logits, k, S, renorm):
    import extreme_quantized_moe_amd as m
    r = m.route_sort(logits.cuda(), k, S, renorm)
    torch.cuda.synchronize()
    ref = oracle.route_ref(logits.numpy(), k, S, renorm)
    np.testing.assert_array_equal(to_np(r["ids"]), ref["ids"])
    np.testing.assert_array_equal(to_np(r["offsets"]), ref["offsets"])
    np.testing.assert_array_equal(to_np(r["sorted_pairs"]), ref["sorted_pairs"])
    np.testing.assert_array_equal(to_np(r["pair_pos"]), ref["pair_pos"])
    np.testing.assert_allclose(to_np(r["w"]), ref["w"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(to_np(r["slot_w"]), ref["slot_w"].reshape(-1), rtol=1e-6, atol=0)


@pytest.mark.parametrize("cfg", [C2, C3, C4], ids=["C2", "C3", "C4"])
def test_route_configs(cfg):
    _check(synth.gen_logits(cfg), cfg.k, cfg.S, cfg.renormalize)


@pytest.mark.parametrize("T,E,k,S,renorm", [
    (1, 8, 2, 0, True), (257, 8, 2, 0, True), (255, 64, 6, 2, False), (513, 256, 8, 0, True),
    (1000, 16, 1, 1, False), (300, 240, 8, 8, True),
    (200, 250, 4, 6, True), (50, 12, 3, 1, False), (256, 32, 4, 0, False)])
def test_route_shapes(T, E, k, S, renorm):
    g = torch.Generator().manual_seed(T * 7 + E)
    _check(torch.randn((T, E), generator=g), k, S, renorm)


@pytest.mark.parametrize("T", [64, 700])
def test_route_ties(T):
    g = torch.Generator().manual_seed(T)
    logits = torch.randint(-2, 3, (T, 8), generator=g).float()
    _check(logits, 3, 1, True)


@pytest.mark.parametrize("T,E,k,S", [(64, 8, 2, 2), (200, 16, 2, 1), (256, 5, 1, 3), (300, 16, 2, 2)])
def test_route_ties_top2_kernel(T, E, k, S):
    """Top-1/top-2 routing with up to four slots per token runs on the router
    instantiation unrolled for two picks and four slots (one and several
    token blocks); integer logits make ties common."""
    g = torch.Generator().manual_seed(T * 3 + E + S)
    logits = torch.randint(-2, 3, (T, E), generator=g).float()
    _check(logits, k, S, True)


@pytest.mark.parametrize("T,E,k,S", [(256, 64, 6, 2), (100, 32, 4, 0)])
def test_route_ties_four_lanes(T, E, k, S):
    """More than 16 experts: four threads per token, each with its own top-k
    over a quarter of the row, merged by (larger value, then lower id).
    Integer logits make ties within and across the quarters common."""
    g = torch.Generator().manual_seed(T + E)
    logits = torch.randint(-2, 3, (T, E), generator=g).float()
    _check(logits, k, S, False)


def test_route_all_to_one_expert():
    logits = torch.full((300, 8), -5.0)
    logits[:, 3] = 5.0
    _check(logits, 1, 0, True)


def test_route_deterministic():
    import extreme_quantized_moe_amd as m
    lg = synth.gen_logits(C3).cuda()
    a = m.route_sort(lg, 2, 0, True)
    b = m.route_sort(lg, 2, 0, True)
    for key in a:
        assert torch.equal(a[key], b[key])
