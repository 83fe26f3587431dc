"""The MoE layer captured into a HIP graph and replayed: every replay, with
new inputs copied into the captured buffers and eager library work run
between replays, must equal the eager layer on the same inputs bit for bit
(the path is deterministic).  The library allocates, synchronizes and
clears nothing inside its calls, so a caller may capture them as they are;
this is the check that such a capture replays correctly."""
import pytest
import torch

from tests.gpu_helpers import make_family

pytestmark = pytest.mark.gpu


def _layer(E, H, F, seed):
    import extreme_quantized_moe_amd as m
    ranks = [16, 32, 64, 8, 24, 40, 0, 56][:E]
    w1, _ = make_family(seed, E, F, H, ranks)
    w3, _ = make_family(seed + 1, E, F, H, ranks)
    w2, _ = make_family(seed + 2, E, H, F, ranks)
    return m.MoELayer(w1, w3, w2, E, 2, 0, True)


def _inputs(T, H, E, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g).half().cuda()
    logits = torch.randn((T, E), generator=g).cuda()
    return x, logits


@pytest.mark.parametrize("T", [16, 300])   # small-M path; tile path (experts average 75 rows)
def test_layer_graph_replays_match_eager(T):
    E, H, F = 8, 256, 512
    layer = _layer(E, H, F, 70 + T)
    cases = [_inputs(T, H, E, 1000 * T + i) for i in range(3)]
    want = [layer.forward(x, lg).clone() for x, lg in cases]
    torch.cuda.synchronize()

    x_s = torch.empty_like(cases[0][0])
    lg_s = torch.empty_like(cases[0][1])
    x_s.copy_(cases[0][0])
    lg_s.copy_(cases[0][1])
    layer.forward(x_s, lg_s)                     # warm-up on the same buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_s = layer.forward(x_s, lg_s)
    torch.cuda.synchronize()

    other = _inputs(T, H, E, 7)
    for rep in range(3):
        for i, (x, lg) in enumerate(cases):
            x_s.copy_(x)
            lg_s.copy_(lg)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_s, want[i]), f"T={T}: replay {rep} of input {i} differs from the eager layer"
            # eager library work between replays (its own buffers)
            layer.forward(*other)
            torch.cuda.synchronize()
