"""The routed W3A16 + low-rank grouped GEMM vs the oracle (float64, unfused):
relative Frobenius error <= 1e-3 and max abs error <= 2e-2 on fp16 outputs,
for both kernel paths, every epilogue, ragged expert sizes and the special
cases of the method (rank 0, zero compensator, zero weights)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import C1
from tests.gpu_helpers import assert_close, make_family, to_np

pytestmark = pytest.mark.gpu

PATHS = {"auto": 0, "decode": 1, "prefill": 2}


def _m():
    import extreme_quantized_moe_amd as m
    return m


def test_c1_single_linear_all_paths():
    m = _m()
    d = synth.gen_linear(C1)
    fam = m.Family.from_dense([d["W"].cuda()], [d["A"]], [d["B"]])
    q, s, z = oracle.quantize_rtn_int3(d["W"].numpy())
    ref = oracle.linear_ref(d["X"].numpy(), q, s, z, d["A"].numpy(), d["B"].numpy())
    x = d["X"].cuda()
    offsets = torch.tensor([0, C1.M], dtype=torch.int32, device="cuda")
    for name, path in PATHS.items():
        y = torch.empty((C1.M, C1.N), dtype=torch.float16, device="cuda")
        m.moe_w3a16_lowrank_gemm((fam,), x, offsets, C1.M, m.EPI_NONE, y, path=path)
        torch.cuda.synchronize()
        assert_close(to_np(y), ref, f"C1 {name}")
    # the compensator matters at this tolerance: dropping it must fail the bar
    ref_nolr = oracle.linear_ref(d["X"].numpy(), q, s, z)
    assert oracle.rel_fro(ref_nolr, ref) > 5e-3


def _route(T, E, k, S, seed, skew=None):
    g = torch.Generator().manual_seed(seed)
    logits = torch.randn((T, E), generator=g)
    if skew is not None:
        logits[:, skew] += 6.0
    return logits


def _moe_case(E, S, N, K, ranks, T, k, epilogue, path, seed, skew=None, zero_w=False, zero_lr=False,
              lr_format="fp16", logits=None, max_rows=None, workspace=None, fill=None):
    m = _m()
    ET = E + S
    if logits is None:
        logits = _route(T, E, k, S, seed, skew)
    r = m.route_sort(logits.cuda(), k, S, True)
    ref_r = oracle.route_ref(logits.numpy(), k, S, True)
    slots = k + S
    P = T * slots
    g = torch.Generator().manual_seed(seed + 1)
    if epilogue == m.EPI_ROUTE_SCALE:
        # down projection input: one row per pair, in sorted order
        x = (torch.randn((P, K), generator=g)).half()
        gather = 0
    else:
        x = (torch.randn((T, K), generator=g)).half()
        gather = slots
    nfam = 2 if epilogue == m.EPI_SWIGLU else 1
    fams, refs = [], []
    for f in range(nfam):
        fam, ref = make_family(seed * 10 + f, ET, N, K, ranks, zero_w=zero_w, zero_lr=zero_lr,
                               lr_format=lr_format)
        fams.append(fam)
        refs.append(ref)
    ydt = torch.float32 if epilogue == m.EPI_ROUTE_SCALE else torch.float16
    if fill is not None:
        y = torch.full((P, N), fill, dtype=ydt, device="cuda")
    elif epilogue == m.EPI_ROUTE_SCALE:
        y = torch.full((P, N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        y = torch.empty((P, N), dtype=torch.float16, device="cuda")
    m.moe_w3a16_lowrank_gemm(tuple(fams), x.cuda(), r["offsets"], P, epilogue, y,
                             sorted_pairs=r["sorted_pairs"], gather_div=gather, slot_w=r["slot_w"],
                             y_rows=P, max_rows_per_expert=T if max_rows is None else max_rows, path=path,
                             workspace=workspace)
    torch.cuda.synchronize()
    got = to_np(y).astype(np.float64)
    xs = x.numpy()
    sp, off = ref_r["sorted_pairs"], ref_r["offsets"]
    want = np.zeros((P, N))
    for e in range(ET):
        seg = sp[off[e]:off[e + 1]]
        if seg.size == 0:
            continue
        rows = xs[seg // slots] if gather else xs[off[e]:off[e + 1]]
        outs = []
        for f in range(nfam):
            q, s, z = refs[f]["q"][e]
            outs.append(oracle.linear_ref(rows, q, s, z, refs[f]["A"][e], refs[f]["B"][e]))
        if epilogue == m.EPI_SWIGLU:
            val = oracle.silu(outs[0]) * outs[1]
        else:
            val = outs[0]
        if epilogue == m.EPI_ROUTE_SCALE:
            want[seg] = val * ref_r["slot_w"].reshape(-1)[seg][:, None]
        else:
            want[off[e]:off[e + 1]] = val
    return got, want


@pytest.mark.parametrize("path", ["decode", "prefill", "auto"])
@pytest.mark.parametrize("epi", ["none", "swiglu", "route"])
def test_small_moe(path, epi):
    m = _m()
    epilogue = {"none": m.EPI_NONE, "swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    # 5 routed + 1 shared experts, ragged ranks (0 .. 64), K = 3 blocks, N = 3 tiles
    got, want = _moe_case(E=5, S=1, N=192, K=384, ranks=[16, 0, 64, 8, 32, 24], T=24, k=2,
                          epilogue=epilogue, path=PATHS[path], seed=3)
    assert_close(got, want, f"small moe {path} {epi}")


@pytest.mark.parametrize("T,path", [(1, "decode"), (7, "decode"), (16, "decode"), (17, "decode"),
                                    (32, "decode"), (33, "auto"), (64, "auto")])
def test_decode_row_counts(T, path):
    m = _m()
    got, want = _moe_case(E=4, S=0, N=128, K=256, ranks=[16, 32, 48, 64], T=T, k=2,
                          epilogue=m.EPI_SWIGLU, path=PATHS[path], seed=T)
    assert_close(got, want, f"{path} T={T}")


def _counts_logits(counts, E):
    """k = 1 logits that send counts[e] consecutive tokens to expert e."""
    T = sum(counts)
    logits = torch.randn((T, E), generator=torch.Generator().manual_seed(T))
    t = 0
    for e, c in enumerate(counts):
        logits[t:t + c, e] += 20.0
        t += c
    return logits


@pytest.mark.parametrize("counts,K,epi,lr", [
    ([8, 9, 1, 0, 16, 7], 256, "swiglu", "fp16"),
    ([8, 9, 1, 0, 16, 7], 384, "route", "int3"),
    ([3, 12], 4096, "swiglu", "fp16"),          # split K
    ([5, 2, 8, 1], 4096, "route", "fp16"),      # split K, experts of at most 8 rows
])
def test_decode_exact_row_counts(counts, K, epi, lr):
    """One decode launch over experts with exactly the given row counts
    (empty, 1, 8, 9, 16 rows; with and without split K)."""
    m = _m()
    E = len(counts)
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=E, S=0, N=128, K=K, ranks=[16, 64, 32, 8, 48, 24][:E], T=sum(counts), k=1,
                          epilogue=epilogue, path=PATHS["decode"], seed=200 + K, lr_format=lr,
                          logits=_counts_logits(counts, E), max_rows=max(counts))
    assert_close(got, want, f"rows {counts} K={K} {epi} {lr}")


@pytest.mark.parametrize("T,epi", [(4, "route"), (16, "swiglu"), (30, "route")])
def test_decode_split_k(T, epi):
    """Few experts and a long K: the small-M kernel splits K over blocks and
    the reduce kernel adds the splits."""
    m = _m()
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=2, S=0, N=128, K=4096, ranks=[16, 64], T=T, k=1,
                          epilogue=epilogue, path=PATHS["decode"], seed=100 + T)
    assert_close(got, want, f"split-K T={T} {epi}")


@pytest.mark.parametrize("T", [100, 300])
def test_prefill_ragged_tiles(T):
    m = _m()
    # skewed routing: expert 2 gets every token (several 128-row tiles + tail),
    # others few or none
    got, want = _moe_case(E=6, S=0, N=256, K=512, ranks=[8, 16, 32, 64, 0, 40], T=T, k=2,
                          epilogue=m.EPI_ROUTE_SCALE, path=PATHS["auto"], seed=T, skew=2)
    assert_close(got, want, f"prefill T={T}")


@pytest.mark.parametrize("T,K,epi", [(400, 1024, "swiglu"), (300, 512, "route"), (200, 2048, "route"),
                                      (400, 512, "swiglu")])
def test_prefill_large_experts(T, K, epi):
    """At least 128 pairs per expert on average: the low-rank pre-pass runs on
    128-row tiles with every rank tile per block (ragged last tiles, a rank-0
    expert, ranks that are not multiples of 16), with K split over blocks at
    K >= 1024 and unsplit at K = 512; the tile GEMM takes 128-row blocks at
    T = 400 (at least 256 pairs per expert) and 64-row blocks below."""
    m = _m()
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=3, S=0, N=128, K=K, ranks=[40, 0, 64], T=T, k=2,
                          epilogue=epilogue, path=PATHS["prefill"], seed=300 + T + K)
    assert_close(got, want, f"large experts T={T} K={K} {epi}")


@pytest.mark.parametrize("epi", ["swiglu", "route"])
def test_prefill_every_tile_shape_256_experts(epi):
    """64-row tile launch over 256 experts whose row counts give every tile
    shape: none (0 rows), one m-tile (1, 16 rows), two (17, 32), four (33,
    63), full tiles alone (64, 128) and full tiles with each shape of
    partial tile (65, 81, 100, 150); the expert table of the gate/up launch
    holds its totals past the last expert."""
    m = _m()
    pattern = [0, 1, 16, 17, 32, 33, 63, 64, 65, 81, 100, 128, 150]
    E = 256
    counts = [pattern[(5 * e) % len(pattern)] for e in range(E)]
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=E, S=0, N=128, K=256, ranks=[16, 0, 64, 8, 32, 24, 48, 40][:4] * 64,
                          T=sum(counts), k=1, epilogue=epilogue, path=PATHS["prefill"], seed=400,
                          logits=_counts_logits(counts, E), max_rows=max(counts))
    assert_close(got, want, f"256 experts, every tile shape, {epi}")


def test_prefill_persistent_several_rounds():
    """The persistent 64-row gate/up launch with several rounds of items per
    block (256 experts of every tile shape, 4 n-tile groups: about 1400
    items for a grid of at most two blocks per CU), so that items are dealt
    in forward and in reverse block order; every output is compared."""
    m = _m()
    pattern = [0, 1, 16, 17, 32, 33, 63, 64, 65, 81, 100, 128, 150]
    E = 256
    counts = [pattern[(7 * e) % len(pattern)] for e in range(E)]
    got, want = _moe_case(E=E, S=0, N=512, K=256, ranks=[16, 32, 0, 8] * 64, T=sum(counts), k=1,
                          epilogue=m.EPI_SWIGLU, path=PATHS["prefill"], seed=410,
                          logits=_counts_logits(counts, E), max_rows=max(counts))
    assert_close(got, want, "persistent launch, several rounds")


@pytest.mark.parametrize("epi,lr", [("swiglu", "fp16"), ("route", "fp16"), ("swiglu", "int3")])
def test_auto_small_matrices_sparse_batch(epi, lr):
    """Automatic path, small matrices, experts averaging under 16 rows with
    one heavy expert (every token): the small-M kernel takes the experts of
    up to 16 rows in one launch, the tile kernel the heavy one."""
    m = _m()
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    ranks = [8, 16, 32, 64, 0, 40, 24, 16, 8, 32, 48, 64, 16, 0, 32, 8]
    got, want = _moe_case(E=16, S=0, N=128, K=256, ranks=ranks, T=40, k=2, epilogue=epilogue,
                          path=PATHS["auto"], seed=77, skew=3, lr_format=lr)
    assert_close(got, want, f"auto sparse {epi} {lr}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_zero_weights_isolate_lowrank(path):
    m = _m()
    got, want = _moe_case(E=3, S=0, N=128, K=256, ranks=[16, 32, 64], T=12, k=2,
                          epilogue=m.EPI_NONE, path=PATHS[path], seed=21, zero_w=True)
    assert np.abs(want).max() > 0
    assert_close(got, want, f"W=0 {path}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_zero_compensator(path):
    m = _m()
    got, want = _moe_case(E=3, S=0, N=128, K=256, ranks=[16, 32, 64], T=12, k=2,
                          epilogue=m.EPI_NONE, path=PATHS[path], seed=22, zero_lr=True)
    assert_close(got, want, f"A=B=0 {path}")


def test_rank_zero_everywhere():
    m = _m()
    got, want = _moe_case(E=2, S=0, N=64, K=128, ranks=[0, 0], T=5, k=1,
                          epilogue=m.EPI_NONE, path=PATHS["auto"], seed=23)
    assert_close(got, want, "rank 0")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_deterministic(path):
    m = _m()
    fam, _ = make_family(40, 4, 128, 1024, [16, 32, 64, 8])
    g = torch.Generator().manual_seed(41)
    T, k = 16, 2
    logits = torch.randn((T, 4), generator=g)
    r = m.route_sort(logits.cuda(), k, 0, True)
    x = torch.randn((T, 1024), generator=g).half().cuda()
    P = T * k
    outs = []
    for _ in range(3):
        y = torch.empty((P, 128), dtype=torch.float32, device="cuda")
        m.moe_w3a16_lowrank_gemm((fam,), x, r["offsets"], P, m.EPI_ROUTE_SCALE, y,
                                 sorted_pairs=r["sorted_pairs"], gather_div=k, slot_w=r["slot_w"],
                                 y_rows=P, max_rows_per_expert=T, path=PATHS[path])
        torch.cuda.synchronize()
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_direct_output_guard_band():
    """Output rows written in place inside a larger sentinel-filled buffer."""
    m = _m()
    fam, ref = make_family(50, 2, 128, 256, [16, 32])
    g = torch.Generator().manual_seed(51)
    T = 8
    x = torch.randn((T, 256), generator=g).half()
    offsets = torch.tensor([0, 3, T], dtype=torch.int32, device="cuda")
    big = torch.full(((T + 4) * 128,), -7.0, dtype=torch.float16, device="cuda")
    y = big[2 * 128:(T + 2) * 128].view(T, 128)
    for path in (1, 2):
        m.moe_w3a16_lowrank_gemm((fam,), x.cuda(), offsets, T, m.EPI_NONE, y, path=path)
        torch.cuda.synchronize()
        assert torch.all(big[:2 * 128] == -7.0) and torch.all(big[(T + 2) * 128:] == -7.0)
        want = np.concatenate([
            oracle.linear_ref(x.numpy()[:3], *ref["q"][0], ref["A"][0], ref["B"][0]),
            oracle.linear_ref(x.numpy()[3:], *ref["q"][1], ref["A"][1], ref["B"][1])])
        assert_close(to_np(y), want, f"in-place path {path}")


def test_workspace_reused_across_different_plans():
    """One zero-initialised workspace serves calls whose plans differ (split
    pre-pass vs not, split-K vs not) in any order."""
    m = _m()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    fam, ref = make_family(60, 3, 128, 1024, [16, 32, 64])
    g = torch.Generator().manual_seed(61)
    for T, path in [(200, 2), (10, 1), (200, 0), (3, 1), (10, 1)]:
        x = torch.randn((T, 1024), generator=g).half()
        cut = [0, T // 3, (2 * T) // 3, T]
        offsets = torch.tensor(cut, dtype=torch.int32, device="cuda")
        y = torch.empty((T, 128), dtype=torch.float16, device="cuda")
        m.moe_w3a16_lowrank_gemm((fam,), x.cuda(), offsets, T, m.EPI_NONE, y,
                                 max_rows_per_expert=T, path=path, workspace=ws)
        torch.cuda.synchronize()
        want = np.concatenate([oracle.linear_ref(x.numpy()[cut[e]:cut[e + 1]], *ref["q"][e],
                                                 ref["A"][e], ref["B"][e]) for e in range(3)])
        assert_close(to_np(y), want, f"reuse T={T} path={path}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_fp16_factors_beyond_rank_are_never_read(path):
    """Columns of U and rows of V at or beyond an expert's rank are never
    read (documented contract): poison them with NaN, the result must not
    change."""
    m = _m()
    E, N, K, ranks = 3, 128, 256, [8, 24, 40]
    fam, _ = make_family(88, E, N, K, ranks)
    g = torch.Generator().manual_seed(89)
    T = 20
    x = torch.randn((T, K), generator=g).half().cuda()
    offsets = torch.tensor([0, 7, 13, T], dtype=torch.int32, device="cuda")

    def run():
        y = torch.empty((T, N), dtype=torch.float16, device="cuda")
        m.moe_w3a16_lowrank_gemm((fam,), x, offsets, T, m.EPI_NONE, y, max_rows_per_expert=T,
                                 path=PATHS[path])
        torch.cuda.synchronize()
        return y.clone()

    clean = run()
    for e, r in enumerate(ranks):
        fam.U[e, :, r:] = float("nan")
        fam.V[e, r:, :] = float("nan")
    dirty = run()
    assert torch.equal(clean, dirty)


@pytest.mark.parametrize("T,epi", [(24, "swiglu"), (40, "route")])
def test_large_matrices_chunked_small_m_plan(T, epi):
    """Large matrices (N K > 2^22) with a row bound of 17..128 and experts
    averaging under 32 rows: the automatic plan runs the one-m-tile small-M
    kernel alone and takes experts above 16 rows in 16-row chunks (no tile
    launch)."""
    m = _m()
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=4, S=0, N=1088, K=4096, ranks=[16, 64, 0, 40], T=T, k=2, epilogue=epilogue,
                          path=PATHS["auto"], seed=500 + T, skew=1)
    assert_close(got, want, f"chunked small-M plan T={T} {epi}")


@pytest.mark.parametrize("epi", ["swiglu", "route"])
def test_row_bound_too_small_chunks_rows(epi):
    """A caller bound below the real rows per expert, small-M plan without
    split K: the kernel takes the heavier experts in 16-row chunks, so every
    row is still correct."""
    m = _m()
    E, N, K, T, k = 4, 128, 256, 40, 2
    e_epi = m.EPI_SWIGLU if epi == "swiglu" else m.EPI_ROUTE_SCALE
    got, want = _moe_case(E, 0, N, K, [16] * E, T, k, e_epi, PATHS["auto"], 91, skew=0, max_rows=8, fill=0.0)
    ref_r = oracle.route_ref(_route(T, E, k, 0, 91, 0).numpy(), k, 0, True)
    rows = np.diff(ref_r["offsets"])
    assert rows.max() > 32 and rows.min() <= 16, rows    # one, two and three chunks
    assert_close(got, want, f"row bound 8, experts of {rows.tolist()} rows, {epi}")


@pytest.mark.parametrize("epi", ["swiglu", "route"])
def test_row_bound_too_small_poisons_rows(epi):
    """A caller bound below the real rows per expert with a split-K small-M
    plan (long K, few items; its partial sums are kept per expert, so it does
    not chunk): the rows of the experts above its 16 rows have no kernel and
    must come back as NaN, not as whatever the output held, while every other
    row is correct."""
    m = _m()
    E, N, K, T, k = 3, 128, 4096, 40, 1
    e_epi = m.EPI_SWIGLU if epi == "swiglu" else m.EPI_ROUTE_SCALE
    counts = [25, 9, 6]
    got, want = _moe_case(E, 0, N, K, [16] * E, T, k, e_epi, PATHS["auto"], 92, max_rows=8, fill=0.0,
                          logits=_counts_logits(counts, E))
    ref_r = oracle.route_ref(_counts_logits(counts, E).numpy(), k, 0, True)
    off, sp = ref_r["offsets"], ref_r["sorted_pairs"]
    rows = np.diff(off)
    assert rows.tolist() == counts, rows
    for e in range(E):
        idx = sp[off[e]:off[e + 1]] if e_epi == m.EPI_ROUTE_SCALE else np.arange(off[e], off[e + 1])
        if rows[e] > 16:
            assert np.all(np.isnan(got[idx])), f"expert {e} ({rows[e]} rows): rows not poisoned"
        else:
            assert_close(got[idx], want[idx], f"expert {e} ({rows[e]} rows) next to a poisoned expert")