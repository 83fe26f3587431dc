"""Shared helpers of the GPU parity tests: build the same seeded inputs for
the oracle (CPU, float64) and the library (GPU), and compare."""
import numpy as np
import torch

import oracle

REL_FRO_TOL = 1e-3
MAX_ABS_TOL = 2e-2


def have_gpu():
    return torch.cuda.is_available()


def to_np(t):
    return t.detach().cpu().numpy()


def assert_close(got, ref, what, rel=REL_FRO_TOL, mabs=MAX_ABS_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rf = oracle.rel_fro(got, ref)
    ma = oracle.max_abs(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert rf <= rel and ma <= mabs, f"{what}: rel_fro={rf:.3e} (tol {rel}) max_abs={ma:.3e} (tol {mabs})"
    return rf, ma


def make_family(rng_seed, E, N, K, ranks, w_sigma=0.02, lr_sigma=0.01, device="cuda",
                zero_w=False, zero_lr=False, lr_format="fp16"):
    """Random fp32 weights + fp16 compensators for E experts (CPU torch
    generator), the library Family built from them on the GPU, and the
    oracle's own quantization of the same weights.  With lr_format "int3" the
    library quantizes the factors too, and the reference factors are the
    oracle's dequantized int3 factors."""
    from extreme_quantized_moe_amd import Family
    g = torch.Generator().manual_seed(rng_seed)
    Ws, As, Bs, q = [], [], [], []
    for e in range(E):
        W = torch.randn((N, K), generator=g) * w_sigma
        if zero_w:
            W.zero_()
        r = ranks[e]
        A = (torch.randn((K, r), generator=g) * lr_sigma).half()
        B = (torch.randn((r, N), generator=g) * lr_sigma).half()
        if zero_lr:
            A.zero_()
            B.zero_()
        Ws.append(W)
        As.append(A)
        Bs.append(B)
        q.append(oracle.quantize_rtn_int3(W.numpy()))
    fam = Family.from_dense([w.to(device) for w in Ws], As, Bs,
                            max_rank=max(max(ranks), 0), lr_format=lr_format)
    A_ref, B_ref = [a.numpy() for a in As], [b.numpy() for b in Bs]
    if lr_format == "int3":
        deq = [oracle.dequant_compensator(oracle.quantize_compensator(a, b)) for a, b in zip(A_ref, B_ref)]
        A_ref, B_ref = [d[0] for d in deq], [d[1] for d in deq]
    return fam, {"W": Ws, "A": A_ref, "B": B_ref, "q": q}
