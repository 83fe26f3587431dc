"""The whole layer at the full workload sizes, in the launch configuration the
benchmark times (bench.Layer: prebuilt descriptors, separate low-rank
pre-pass, AUTO path), against the float64 oracle on sampled outputs:

* the SwiGLU intermediate G for every pair and a sample of its columns (the
  oracle needs only those rows of W1 and W3);
* the layer output for a sample of tokens and of output columns (the oracle
  recomputes the sampled tokens' expert FFNs in full width, and only the
  sampled rows of W2).

Tolerance as everywhere: relative Frobenius error <= 1e-3 and max abs error
<= 2e-2.  Weights and activations are generated once on the GPU and copied
to the host for the oracle (the seeded generators give device-dependent
streams)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs as SC
from tests.gpu_helpers import assert_close

pytestmark = pytest.mark.gpu


def _run_layer(cfg, layer, lr_format="fp16"):
    import bench
    import extreme_quantized_moe_amd as m
    X = synth.gen_tokens(cfg, 0, device="cuda")
    logits = synth.gen_logits(cfg, layer, device="cuda")
    lay = bench.Layer(m, cfg, layer, X, logits, 0, lr_format=lr_format)
    lay.ws = torch.zeros(lay.ws_need, dtype=torch.uint8, device="cuda")
    lay.step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return lay


def _cols(n, count, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=count, replace=False))


def _quantize_rows(W, rows):
    return oracle.quantize_rtn_int3(W[rows].astype(np.float32))


def _expert_host(cfg, layer, e, rank, which, lr_format="fp16"):
    """One expert's tensors on the host; with int3 factors the compensators
    are replaced by the oracle's dequantized int3 factors."""
    d = synth.gen_expert(cfg, layer, e, rank, device="cuda", which=which)
    d = {k: v.cpu().numpy() for k, v in d.items()}
    if lr_format == "int3":
        for a, b in (("A1", "B1"), ("A3", "B3"), ("A2", "B2")):
            if a in d:
                d[a], d[b] = oracle.dequant_compensator(oracle.quantize_compensator(d[a], d[b]))
    return d


def _check_g(cfg, layer, lay, ncols, seed, lr_format="fp16"):
    """G[pair][n] = silu(h1) * h3 for every pair and sampled columns n."""
    cols = _cols(cfg.F, ncols, seed)
    route = oracle.route_ref(lay.logits.cpu().numpy(), cfg.k, cfg.S, cfg.renormalize)
    sp, off = route["sorted_pairs"], route["offsets"]
    X = lay.X.cpu().numpy().astype(np.float64)
    got = lay.G.cpu().numpy().astype(np.float64)[:, cols]
    want = np.zeros_like(got)
    for e in range(cfg.E + cfg.S):
        if off[e + 1] == off[e]:
            continue
        d = _expert_host(cfg, layer, e, lay.ranks[e], ("W1", "W3"), lr_format)
        rows = X[sp[off[e]:off[e + 1]] // cfg.slots]
        h = []
        for n, a, b in (("W1", "A1", "B1"), ("W3", "A3", "B3")):
            q, s, z = _quantize_rows(d[n], cols)
            h.append(oracle.linear_ref(rows, q, s, z, d[a], d[b][:, cols]))
        want[off[e]:off[e + 1]] = oracle.silu(h[0]) * h[1]
    rf, ma = assert_close(got, want, f"{cfg.name} G (all pairs, {ncols} columns, {lr_format} factors)")
    print(f"{cfg.name} G (all pairs, {ncols} columns, {lr_format} factors): rel_fro {rf:.2e} max_abs {ma:.2e}")


def _check_out(cfg, layer, lay, toks, ncols, seed, lr_format="fp16"):
    """out[t][c] for sampled tokens t and output columns c."""
    cols = _cols(cfg.H, ncols, seed) if ncols < cfg.H else np.arange(cfg.H)
    X = lay.X.cpu().numpy()[toks].astype(np.float64)
    logits = lay.logits.cpu().numpy()[toks]

    def get_expert(e):
        d = _expert_host(cfg, layer, e, lay.ranks[e], ("W1", "W3", "W2"), lr_format)
        qe = {n: oracle.quantize_rtn_int3(d[n]) for n in ("W1", "W3")}
        qe["W2"] = _quantize_rows(d["W2"], cols)
        qe.update({n: d[n] for n in ("A1", "B1", "A3", "B3", "A2")})
        qe["B2"] = d["B2"][:, cols]
        return qe

    # get_expert already keeps only the sampled rows of W2 (and columns of B2)
    ref = oracle.moe_layer_ref(X, logits, get_expert, cfg.k, cfg.S, cfg.renormalize,
                               out_cols=np.arange(len(cols)))
    got = lay.out.cpu().numpy().astype(np.float64)[toks][:, cols]
    rf, ma = assert_close(got, ref["out"], f"{cfg.name} out ({len(toks)} tokens, {len(cols)} columns, {lr_format} factors)")
    print(f"{cfg.name} out ({len(toks)} tokens, {len(cols)} columns, {lr_format} factors): rel_fro {rf:.2e} max_abs {ma:.2e}")


def _check_tokens_full(cfg, layer, lay, toks, what):
    """Every column of G for every pair of the tokens toks, and every column
    of their layer output (the oracle recomputes those tokens' expert FFNs in
    full).  Returns the (rel_fro, max_abs) of both checks."""
    toks = np.asarray(sorted(set(int(t) for t in toks)))
    X = lay.X.cpu().numpy()[toks].astype(np.float64)
    logits = lay.logits.cpu().numpy()[toks]

    def get_expert(e):
        d = _expert_host(cfg, layer, e, lay.ranks[e], ("W1", "W3", "W2"))
        return oracle.quantize_expert(d)

    ref = oracle.moe_layer_ref(X, logits, get_expert, cfg.k, cfg.S, cfg.renormalize)
    pair_pos = lay.route["pair_pos"].cpu().numpy()
    G = lay.G.cpu().numpy()
    s_loc = sorted(ref["g_pair"])
    got_g = np.stack([G[pair_pos[toks[s // cfg.slots] * cfg.slots + s % cfg.slots]] for s in s_loc])
    want_g = np.stack([ref["g_pair"][s] for s in s_loc])
    g_err = assert_close(got_g, want_g, f"{what}: G ({len(s_loc)} pairs, all {cfg.F} columns)")
    got_o = lay.out.cpu().numpy().astype(np.float64)[toks]
    o_err = assert_close(got_o, ref["out"], f"{what}: out ({len(toks)} tokens, all {cfg.H} columns)")
    print(f"{what}: G rel_fro {g_err[0]:.2e} max_abs {g_err[1]:.2e}; out rel_fro {o_err[0]:.2e} "
          f"max_abs {o_err[1]:.2e} (bounds 1e-3, 2e-2)")
    return g_err, o_err


def test_c2_full_decode_layer():
    cfg = SC.get_config("C2")
    lay = _run_layer(cfg, 0)
    _check_g(cfg, 0, lay, 96, seed=1)
    _check_out(cfg, 0, lay, np.arange(cfg.T), 512, seed=2)


def test_c4_full_layer_all_outputs():
    """DeepSeekMoE-shaped: 64 routed (Zipf-skewed) + 2 shared experts; light
    experts take the decode kernels, heavy ones the tile kernel."""
    cfg = SC.get_config("C4")
    lay = _run_layer(cfg, 0)
    _check_g(cfg, 0, lay, 64, seed=3)
    _check_out(cfg, 0, lay, np.arange(cfg.T), cfg.H, seed=4)


def test_c3_full_prefill_layer_sampled():
    cfg = SC.get_config("C3")
    lay = _run_layer(cfg, 0)
    _check_g(cfg, 0, lay, 16, seed=5)
    _check_out(cfg, 0, lay, [0, 1234, 2900, cfg.T - 1], 256, seed=6)


@pytest.mark.timeout(900)
def test_c3_full_prefill_tile_edges():
    """C3 at full size: for every 128-row tile of every expert (the tile
    kernel's row blocks at prefill), the pairs on its first and last row --
    all columns of their G rows, and all output columns of their tokens
    (which brings in every other pair of those tokens as well)."""
    cfg = SC.get_config("C3")
    lay = _run_layer(cfg, 0)
    route = oracle.route_ref(lay.logits.cpu().numpy(), cfg.k, cfg.S, cfg.renormalize)
    sp, off = route["sorted_pairs"], route["offsets"]
    np.testing.assert_array_equal(lay.route["offsets"].cpu().numpy(), off)
    toks = []
    for e in range(cfg.E + cfg.S):
        M = int(off[e + 1] - off[e])
        for m0 in range(0, M, 128):
            for m in (m0, min(m0 + 127, M - 1)):
                toks.append(int(sp[off[e] + m]) // cfg.slots)
    _check_tokens_full(cfg, 0, lay, toks, "C3 tile edges")


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_c5_layer_at_batch(T):
    """One layer of the 32-layer stack at each batch size the benchmark sweeps:
    1 (one token, two experts), 8, 32 (two-m-tile decode items at K = 14336)
    and 64 (both kernels)."""
    cfg = SC.get_config("C5").with_(T=T)
    lay = _run_layer(cfg, 7)
    _check_g(cfg, 7, lay, 32, seed=7)
    _check_out(cfg, 7, lay, [0] if T == 1 else sorted({1, 5, T // 2, T - 1}), 256, seed=8)


def test_c2_full_decode_layer_int3_factors():
    """C2 with the compensators stored as int3 (V rows in groups of 64 along
    K, U rows in one group of r), quantized and packed on the GPU."""
    cfg = SC.get_config("C2")
    lay = _run_layer(cfg, 0, "int3")
    _check_g(cfg, 0, lay, 96, seed=11, lr_format="int3")
    _check_out(cfg, 0, lay, np.arange(cfg.T), 512, seed=12, lr_format="int3")


def test_c4_full_layer_int3_factors():
    cfg = SC.get_config("C4")
    lay = _run_layer(cfg, 0, "int3")
    _check_g(cfg, 0, lay, 64, seed=13, lr_format="int3")
    _check_out(cfg, 0, lay, np.arange(cfg.T), cfg.H, seed=14, lr_format="int3")
