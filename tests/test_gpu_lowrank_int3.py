"""int3 compensator factors on the GPU vs the oracle: the grouped quantizer
and the two factor layouts bit-exact, and the routed GEMM with int3 factors
within the usual bar (relative Frobenius error <= 1e-3, max abs <= 2e-2) on
both kernel paths, every epilogue, ragged ranks, split-K, and with the layout
padding overwritten by garbage (it must never be read into a result)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import C1
from tests.gpu_helpers import assert_close, make_family, to_np
from tests.test_gpu_gemm import PATHS, _moe_case

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _m():
    import extreme_quantized_moe_amd as m
    return m


@pytest.mark.parametrize("rows,K,group", [(64, 8, 8), (128, 16, 16), (64, 24, 24), (200, 32, 32),
                                          (96, 64, 64), (16, 4096, 64), (64, 40, 40), (32, 96, 32)])
def test_grouped_quantizer_bit_exact(rows, K, group):
    m = _m()
    g = torch.Generator().manual_seed(rows + K + group)
    W = (torch.randn((rows, K), generator=g) * 0.01).half().float()   # factors are fp16 values
    W[0, :group] = 0.0                                                 # a constant group
    c, s, z = m.quantize_rtn_int3(W.cuda(), group)
    torch.cuda.synchronize()
    qr, sr, zr = oracle.quantize_rtn_int3(W.numpy().astype(np.float64), group)
    np.testing.assert_array_equal(to_np(c), qr)
    np.testing.assert_array_equal(to_np(s).view(np.uint16), sr.view(np.uint16))
    np.testing.assert_array_equal(to_np(z).view(np.uint16), zr.view(np.uint16))


def test_grouped_quantizer_golden_u_row():
    m = _m()
    c = json.load(open(os.path.join(GOLD, "compensator_cases.json")))["u_row"]
    W = torch.tensor([c["values"]], dtype=torch.float32)
    q, s, z = m.quantize_rtn_int3(W.cuda(), 8)
    assert to_np(q)[0].tolist() == c["codes"]
    assert int(to_np(s).view(np.uint16)[0, 0]) == c["scale_bits"]
    assert int(to_np(z).view(np.uint16)[0, 0]) == c["zero_bits"]


def _rand_factor_codes(rng, N, K, r):
    v = (rng.integers(0, 8, (r, K), dtype=np.uint8), rng.uniform(1e-3, 1e-2, (r, K // 64)).astype(np.float16),
         rng.uniform(0, 7, (r, K // 64)).astype(np.float16))
    u = (rng.integers(0, 8, (N, r), dtype=np.uint8), rng.uniform(1e-3, 1e-2, N).astype(np.float16),
         rng.uniform(0, 7, N).astype(np.float16))
    return v, u


@pytest.mark.parametrize("N,K,r,R", [(64, 128, 16, 16), (128, 256, 8, 16), (192, 384, 24, 32),
                                     (64, 128, 64, 64), (128, 256, 40, 64), (64, 128, 0, 32)])
def test_pack_lr_bit_exact(N, K, r, R):
    m = _m()
    rng = np.random.default_rng(N + K + r)
    v, u = _rand_factor_codes(rng, N, K, r)
    cu = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()
    vq, vsz, uq, usz = m.pack_lr_int3(tuple(cu(t) for t in v) if r else None,
                                      tuple(cu(t) for t in u) if r else None, N, K, r, R)
    torch.cuda.synchronize()
    wv, sv = oracle.pack_lr_v(v[0], v[1], v[2], R)
    wu, su = oracle.pack_lr_u(u[0], u[1], u[2], R)
    np.testing.assert_array_equal(to_np(vq).view(np.uint32), wv)
    np.testing.assert_array_equal(to_np(vsz).view(np.uint32), sv)
    np.testing.assert_array_equal(to_np(uq).view(np.uint32), wu)
    np.testing.assert_array_equal(to_np(usz).view(np.uint32), su)


def test_pack_lr_golden_words():
    m = _m()
    cases = json.load(open(os.path.join(GOLD, "compensator_cases.json")))
    for c in cases["v_layout"]:
        R, K = c["max_rank"], c["K"]
        codes = np.zeros((R, K), np.uint8)
        for j, k, val in c["set"]:
            codes[j, k] = val
        ones = torch.ones((R, K // 64), dtype=torch.float16, device="cuda")
        nil = torch.zeros_like(ones)
        u = (torch.zeros((64, R), dtype=torch.uint8, device="cuda"), torch.ones(64, dtype=torch.float16,
             device="cuda"), torch.zeros(64, dtype=torch.float16, device="cuda"))
        vq, _, _, _ = m.pack_lr_int3((torch.from_numpy(codes).cuda(), ones, nil), u, 64, K, R, R)
        w = to_np(vq).view(np.uint32)
        assert {int(i): int(w[i]) for i in np.nonzero(w)[0]} == {int(i): v for i, v in c["expect"].items()}, c["why"]
    for c in cases["u_layout"]:
        N, R = c["N"], c["max_rank"]
        codes = np.zeros((N, R), np.uint8)
        for n, j, val in c["set"]:
            codes[n, j] = val
        v = (torch.zeros((R, 128), dtype=torch.uint8, device="cuda"), torch.ones((R, 2), dtype=torch.float16,
             device="cuda"), torch.zeros((R, 2), dtype=torch.float16, device="cuda"))
        u = (torch.from_numpy(codes).cuda(), torch.ones(N, dtype=torch.float16, device="cuda"),
             torch.zeros(N, dtype=torch.float16, device="cuda"))
        _, _, uq, _ = m.pack_lr_int3(v, u, N, 128, R, R)
        w = to_np(uq).view(np.uint32)
        assert {int(i): int(w[i]) for i in np.nonzero(w)[0]} == {int(i): v for i, v in c["expect"].items()}, c["why"]


def test_family_preparation_matches_oracle():
    """Family.from_dense(lr_format="int3") = oracle quantization + oracle
    packing of the same fp16 factors, word for word, for every expert."""
    fam, _ = make_family(7, 3, 128, 256, [16, 0, 40], lr_format="int3")
    g = torch.Generator().manual_seed(7)
    As, Bs = [], []
    for r in [16, 0, 40]:
        torch.randn((128, 256), generator=g)                  # W (same draw order as make_family)
        As.append((torch.randn((256, r), generator=g) * 0.01).half().numpy())
        Bs.append((torch.randn((r, 128), generator=g) * 0.01).half().numpy())
    Vq, Vsz, Uq, Usz = (to_np(t).view(np.uint32) for t in fam.lrq)
    nv, nvs, nu, nus = oracle.lr_v_words(40, 256), oracle.lr_v_sz_words(40, 256), oracle.lr_u_words(128, 40), 128
    for e, (A, B) in enumerate(zip(As, Bs)):
        q = oracle.quantize_compensator(A, B)
        wv, sv = oracle.pack_lr_v(q["v_codes"], q["v_scale"], q["v_zero"], 40)
        wu, su = oracle.pack_lr_u(q["u_codes"], q["u_scale"], q["u_zero"], 40)
        np.testing.assert_array_equal(Vq[e * nv:(e + 1) * nv], wv)
        np.testing.assert_array_equal(Vsz[e * nvs:(e + 1) * nvs], sv)
        np.testing.assert_array_equal(Uq[e * nu:(e + 1) * nu], wu)
        np.testing.assert_array_equal(Usz[e * nus:(e + 1) * nus], su)


def test_c1_single_linear_int3_factors():
    m = _m()
    d = synth.gen_linear(C1)
    fam = m.Family.from_dense([d["W"].cuda()], [d["A"]], [d["B"]], lr_format="int3")
    q, s, z = oracle.quantize_rtn_int3(d["W"].numpy())
    Ad, Bd = oracle.dequant_compensator(oracle.quantize_compensator(d["A"].numpy(), d["B"].numpy()))
    ref = oracle.linear_ref(d["X"].numpy(), q, s, z, Ad, Bd)
    x = d["X"].cuda()
    offsets = torch.tensor([0, C1.M], dtype=torch.int32, device="cuda")
    for name, path in PATHS.items():
        y = torch.empty((C1.M, C1.N), dtype=torch.float16, device="cuda")
        m.moe_w3a16_lowrank_gemm((fam,), x, offsets, C1.M, m.EPI_NONE, y, path=path)
        torch.cuda.synchronize()
        assert_close(to_np(y), ref, f"C1 int3 factors {name}")
    # the factor rounding is visible at this tolerance: the fp16-factor result
    # is not an acceptable answer for the int3 call
    ref_fp16 = oracle.linear_ref(d["X"].numpy(), q, s, z, d["A"].numpy(), d["B"].numpy())
    assert oracle.rel_fro(ref_fp16, ref) > 2e-3


@pytest.mark.parametrize("path", ["decode", "prefill", "auto"])
@pytest.mark.parametrize("epi", ["none", "swiglu", "route"])
def test_small_moe_int3_factors(path, epi):
    m = _m()
    epilogue = {"none": m.EPI_NONE, "swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=5, S=1, N=192, K=384, ranks=[16, 0, 64, 8, 32, 24], T=24, k=2,
                          epilogue=epilogue, path=PATHS[path], seed=3, lr_format="int3")
    assert_close(got, want, f"small moe int3 {path} {epi}")


@pytest.mark.parametrize("T,path", [(1, "decode"), (16, "decode"), (17, "decode"), (32, "decode"),
                                    (64, "auto")])
def test_decode_row_counts_int3(T, path):
    m = _m()
    got, want = _moe_case(E=4, S=0, N=128, K=256, ranks=[16, 32, 48, 64], T=T, k=2,
                          epilogue=m.EPI_SWIGLU, path=PATHS[path], seed=T, lr_format="int3")
    assert_close(got, want, f"int3 {path} T={T}")


@pytest.mark.parametrize("T,epi", [(4, "route"), (30, "swiglu")])
def test_decode_split_k_int3(T, epi):
    m = _m()
    epilogue = {"swiglu": m.EPI_SWIGLU, "route": m.EPI_ROUTE_SCALE}[epi]
    got, want = _moe_case(E=2, S=0, N=128, K=4096, ranks=[16, 64], T=T, k=1,
                          epilogue=epilogue, path=PATHS["decode"], seed=100 + T, lr_format="int3")
    assert_close(got, want, f"int3 split-K T={T} {epi}")


@pytest.mark.parametrize("T", [100, 300])
def test_prefill_ragged_tiles_int3(T):
    m = _m()
    got, want = _moe_case(E=6, S=0, N=256, K=512, ranks=[8, 16, 32, 64, 0, 40], T=T, k=2,
                          epilogue=m.EPI_ROUTE_SCALE, path=PATHS["auto"], seed=T, skew=2, lr_format="int3")
    assert_close(got, want, f"int3 prefill T={T}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_zero_weights_isolate_int3_lowrank(path):
    m = _m()
    got, want = _moe_case(E=3, S=0, N=128, K=256, ranks=[16, 32, 64], T=12, k=2,
                          epilogue=m.EPI_NONE, path=PATHS[path], seed=21, zero_w=True, lr_format="int3")
    assert np.abs(want).max() > 0
    assert_close(got, want, f"W=0 int3 {path}")


def _padding_masks(N, K, ranks, R):
    """Boolean masks of the padding words (ranks at or beyond each expert's
    rank, including the layouts' round-up rows) of the concatenated Vq / Vsz /
    Uq arrays: pack all-sevens codes and a marker scale in the real ranks
    with the oracle layouts; every other word is padding."""
    mv, ms, mu = [], [], []
    for r in ranks:
        vc = np.zeros((R, K), np.uint8)
        vc[:r] = 7
        s = np.full((R, K // 64), 0.5, np.float16)           # 0x3800
        w, sz = oracle.pack_lr_v(vc[:r], s[:r], np.zeros_like(s[:r]), R)
        mv.append(w != 0xFFFFFFFF)
        ms.append(sz != 0x3800)
        uc = np.full((N, r), 7, np.uint8)
        w, _ = oracle.pack_lr_u(uc, np.ones(N, np.float16), np.zeros(N, np.float16), R)
        mu.append(w != 0xFFFFFFFF)
    return np.concatenate(mv), np.concatenate(ms), np.concatenate(mu)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_padding_is_never_read_into_results(path):
    m = _m()
    E, N, K, ranks = 3, 128, 256, [8, 24, 40]
    fam, _ = make_family(77, E, N, K, ranks, lr_format="int3")
    g = torch.Generator().manual_seed(78)
    T = 20
    x = torch.randn((T, K), generator=g).half().cuda()
    cut = [0, 7, 13, T]
    offsets = torch.tensor(cut, dtype=torch.int32, device="cuda")

    def run():
        y = torch.empty((T, N), dtype=torch.float16, device="cuda")
        m.moe_w3a16_lowrank_gemm((fam,), x, offsets, T, m.EPI_NONE, y, max_rows_per_expert=T,
                                 path=PATHS[path])
        torch.cuda.synchronize()
        return y.clone()

    clean = run()
    mv, ms, mu = _padding_masks(N, K, ranks, 40)
    Vq, Vsz, Uq, Usz = fam.lrq
    assert mv.sum() > 0 and mu.sum() > 0 and ms.sum() > 0
    rng = np.random.default_rng(79)
    for t, mask, val in ((Vq, mv, None), (Vsz, ms, 0x7FFF7FFF), (Uq, mu, None)):
        h = to_np(t).view(np.uint32).copy()
        h[mask] = rng.integers(0, 2 ** 32, int(mask.sum()), dtype=np.uint64).astype(np.uint32) if val is None else val
        t.copy_(torch.from_numpy(h.view(np.int32)).cuda())
    dirty = run()
    assert torch.equal(clean, dirty)
