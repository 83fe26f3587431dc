"""Compensated int3 linear, SwiGLU expert FFN and the routed MoE layer
(oracle side, float64, unfused).

[talk] MiLo Algorithm: the weight used at inference is the quantized weight
plus a low-rank compensator, W_out = W_quant + U V with U of shape (out x R) and
V of shape (R x in).  The workloads give the compensator as A (K x r) and
B (r x N), i.e. U = B^T and V = A^T, so for activations X (M x K):

    Y = X deq(Wq)^T + (X A) B                      (= X (deq(Wq) + (A B)^T)^T)

[talk] MiLo Kernel: the fused kernel computes the same product as a separate
dequantization followed by an fp16 GEMM; the oracle is that unfused definition.

Expert FFN (SwiGLU, compensator added before the activation because it is part
of the weight):
    h1 = linear(x; W1), h3 = linear(x; W3), g = silu(h1) * h3, y = linear(g; W2)
    silu(u) = u / (1 + exp(-u))
MoE layer ([talk] Background): out[t] = sum_j w[t, j] * y[t, j] over the
token's routed slots (and shared slots with weight 1), summed in slot order.
"""
import numpy as np

from .quant import dequant_int3, quantize_rtn_int3
from .route import route_ref


def linear_ref(X, codes, scale, zero, A=None, B=None, group=64):
    """X [M][K], codes [N][K], scale/zero [N][K/group], A [K][r], B [r][N] ->
    Y [M][N] float64."""
    X = np.asarray(X).astype(np.float64)
    Wd = dequant_int3(codes, scale, zero, group)
    Y = X @ Wd.T
    if A is not None and B is not None and np.asarray(A).shape[1] > 0:
        A = np.asarray(A).astype(np.float64)
        B = np.asarray(B).astype(np.float64)
        Y = Y + (X @ A) @ B
    return Y


def silu(u):
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


def quantize_expert(exp, group=64, lr_format="fp16"):
    """fp32 expert weights -> dict with (codes, scale, zero) per matrix plus the
    compensators: unchanged (lr_format "fp16"), or quantized to int3 and
    dequantized again (lr_format "int3", oracle.compensator: [talk] MiLo
    Algorithm, last step -- the factors themselves are stored as int3)."""
    from .compensator import dequant_compensator, quantize_compensator
    out = {}
    for n in ("W1", "W3", "W2"):
        if n not in exp:
            continue
        W = exp[n]
        W = W.numpy() if hasattr(W, "numpy") else np.asarray(W)
        out[n] = quantize_rtn_int3(W, group)
    for n in ("A1", "B1", "A3", "B3", "A2", "B2"):
        if n in exp:
            v = exp[n]
            out[n] = v.numpy() if hasattr(v, "numpy") else np.asarray(v)
    if lr_format == "int3":
        for a, b in (("A1", "B1"), ("A3", "B3"), ("A2", "B2")):
            if a in out and b in out:
                out[a], out[b] = dequant_compensator(quantize_compensator(out[a], out[b]))
    elif lr_format != "fp16":
        raise ValueError(f"unknown compensator format {lr_format!r}")
    return out


def expert_ffn_ref(x, qe, group=64, out_cols=None):
    """x [m][H]; qe: quantized expert (see quantize_expert).  Returns (g, y)
    with g [m][F] and y [m][H] (or y [m][len(out_cols)] if out_cols given)."""
    c1, s1, z1 = qe["W1"]
    c3, s3, z3 = qe["W3"]
    c2, s2, z2 = qe["W2"]
    h1 = linear_ref(x, c1, s1, z1, qe.get("A1"), qe.get("B1"), group)
    h3 = linear_ref(x, c3, s3, z3, qe.get("A3"), qe.get("B3"), group)
    g = silu(h1) * h3
    if out_cols is None:
        y = linear_ref(g, c2, s2, z2, qe.get("A2"), qe.get("B2"), group)
    else:
        cols = np.asarray(out_cols)
        B2 = qe.get("B2")
        y = linear_ref(g, c2[cols], s2[cols], z2[cols], qe.get("A2"),
                       None if B2 is None else np.asarray(B2)[:, cols], group)
    return g, y


def moe_layer_ref(X, logits, get_expert, k, S=0, renormalize=True, group=64,
                  out_cols=None, route=None):
    """Routed MoE layer.  get_expert(e) returns the quantized expert e
    (quantize_expert format); it is called once per expert that receives at
    least one pair, so experts can be streamed.

    Returns dict: out [T][H'] float64, y_slot [T*slots][H'] (route-weighted
    per-slot outputs), g_pair {slot index: g row}, route (route_ref dict)."""
    X = np.asarray(X).astype(np.float64)
    T = X.shape[0]
    if route is None:
        route = route_ref(logits, k, S, renormalize)
    slots = k + S
    E_tot = len(route["offsets"]) - 1
    sp, off = route["sorted_pairs"], route["offsets"]
    slot_w = route["slot_w"].reshape(-1)
    H_out = X.shape[1] if out_cols is None else len(out_cols)
    y_slot = np.zeros((T * slots, H_out), dtype=np.float64)
    g_pair = {}
    for e in range(E_tot):
        seg = sp[off[e]:off[e + 1]]
        if seg.size == 0:
            continue
        qe = get_expert(e)
        rows = X[seg // slots]
        g, y = expert_ffn_ref(rows, qe, group, out_cols)
        y_slot[seg] = y * slot_w[seg][:, None]
        for i, s in enumerate(seg):
            g_pair[int(s)] = g[i]
    out = combine_ref(y_slot, T, slots)
    return {"out": out, "y_slot": y_slot, "g_pair": g_pair, "route": route}


def combine_ref(y_slot, T, slots):
    """out[t] = sum over j = 0..slots-1 (in order) of y_slot[t*slots + j]."""
    y = np.asarray(y_slot, dtype=np.float64).reshape(T, slots, -1)
    out = np.zeros((T, y.shape[2]), dtype=np.float64)
    for j in range(slots):
        out += y[:, j]
    return out


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_abs(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
