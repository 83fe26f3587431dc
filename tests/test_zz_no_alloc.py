"""The static-workspace GEMM entry point (milo_moe_w3a16_lowrank_gemm_static,
for callers that cannot allocate) against the workspace entry point, called
through the C ABI: the same descriptor must give bit-identical outputs, on two
calls in a row (the second on a smaller input, so it runs on the scratch the
first one left behind), for the gate/up (SwiGLU) and the down (route-scale)
projections, on the small-M and on the tile path; and an oversized or flagged
descriptor is rejected before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

from tests.gpu_helpers import make_family

pytestmark = pytest.mark.gpu


def _m():
    import extreme_quantized_moe_amd as m
    return m


def _call_both(m, fams, x, r, P, epilogue, T, slots, path):
    L = m._lib
    lib = L.lib()
    ydt = torch.float32 if epilogue == L.EPI_ROUTE_SCALE else torch.float16
    outs = []
    for static in (False, True):
        y = torch.full((P, fams[0].N), 7.0, dtype=ydt, device="cuda")
        d = m.ops.make_gemm_desc(fams, x, r["offsets"], P, epilogue, y, sorted_pairs=r["sorted_pairs"],
                                 gather_div=slots if epilogue == L.EPI_SWIGLU else 0, slot_w=r["slot_w"],
                                 y_rows=P, max_rows_per_expert=T, path=path)
        stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        if static:
            rc = lib.milo_moe_w3a16_lowrank_gemm_static(C.byref(d), stream)
        else:
            nbytes = int(lib.milo_moe_gemm_workspace_bytes(C.byref(d)))
            assert 0 < nbytes <= L.STATIC_WORKSPACE_BYTES, nbytes
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            rc = lib.milo_moe_w3a16_lowrank_gemm(C.byref(d), C.c_void_p(ws.data_ptr()), nbytes, stream)
        assert rc == 0, lib.milo_last_error()
        torch.cuda.synchronize()
        outs.append(y.cpu())
    return outs


@pytest.mark.parametrize("path", [0, 2])
def test_static_workspace_matches_workspace_call(path):
    m = _m()
    E, H, F, k = 8, 256, 512, 2
    for T in (48, 6):             # second call smaller than the first
        g = torch.Generator().manual_seed(T)
        logits = torch.randn((T, E), generator=g)
        r = m.route_sort(logits.cuda(), k, 0, True)
        x = torch.randn((T, H), generator=g).half().cuda()
        slots = k
        P = T * slots
        w1, _ = make_family(1 + T, E, F, H, [16, 32, 8, 64, 16, 0, 32, 64])
        w3, _ = make_family(2 + T, E, F, H, [16, 32, 8, 64, 16, 0, 32, 64])
        w2, _ = make_family(3 + T, E, H, F, [16, 32, 8, 64, 16, 0, 32, 64])
        ga, gb = _call_both(m, (w1, w3), x, r, P, m._lib.EPI_SWIGLU, T, slots, path)
        assert torch.isfinite(ga.float()).all()
        assert torch.equal(ga.view(torch.int16), gb.view(torch.int16)), f"T={T} path={path}: gate/up differs"
        ya, yb = _call_both(m, (w2,), ga.cuda(), r, P, m._lib.EPI_ROUTE_SCALE, T, slots, path)
        assert torch.isfinite(ya).all()
        assert torch.equal(ya.view(torch.int32), yb.view(torch.int32)), f"T={T} path={path}: down differs"


def test_static_workspace_rejects_before_launch():
    m = _m()
    L = m._lib
    lib = L.lib()
    w, _ = make_family(5, 4, 64, 128, [8, 8, 8, 8])
    x = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    offsets = torch.tensor([0, 1, 2, 3, 4], dtype=torch.int32, device="cuda")
    y = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    d = m.ops.make_gemm_desc((w,), x, offsets, 4, L.EPI_NONE, y)
    d.flags = L.GEMM_PREPASS_DONE
    assert lib.milo_moe_w3a16_lowrank_gemm_static(C.byref(d), None) == 6
    # a descriptor whose workspace exceeds the static scratch: num_pairs large
    # on the tile path (low-rank products of 2^20 pairs x 64 ranks x 2 bytes)
    d.flags = 0
    d.num_pairs = 1 << 20
    d.max_rank = 64
    d.path = L.PATH_PREFILL
    need = int(lib.milo_moe_gemm_workspace_bytes(C.byref(d)))
    assert need > L.STATIC_WORKSPACE_BYTES
    assert lib.milo_moe_w3a16_lowrank_gemm_static(C.byref(d), None) == 5
    assert b"static" in lib.milo_last_error()
    torch.cuda.synchronize()
    assert torch.all(y == 0)
