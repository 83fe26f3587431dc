"""Pins for the oracle's compensated linear, expert FFN and MoE layer
(oracle/moe.py): pure-Python loops, exact integer cases, the compensator
identity W_out = W_quant + U V from the MiLo talk write-up (Technical Deep
Dive, MiLo Algorithm), and MoE special cases."""
import math

import numpy as np
import pytest

import oracle


def _rand_q(rng, N, K):
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return oracle.quantize_rtn_int3(W)


def _py_linear(X, q, s, z, A, B):
    """Triple loop, one scalar at a time."""
    M, K = len(X), len(X[0])
    N = len(q)
    r = len(A[0]) if A is not None else 0
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        t = [sum(float(X[m][k]) * float(A[k][j]) for k in range(K)) for j in range(r)]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                g = k // 64
                acc += float(X[m][k]) * ((float(q[n][k]) - float(z[n][g])) * float(s[n][g]))
            for j in range(r):
                acc += t[j] * float(B[j][n])
            Y[m][n] = acc
    return Y


@pytest.mark.parametrize("M,N,K,r", [(1, 3, 64, 0), (2, 5, 64, 2), (4, 8, 128, 4), (3, 2, 128, 8)])
def test_linear_matches_python_loops(M, N, K, r):
    rng = np.random.default_rng(M * 7 + N + K + r)
    X = rng.standard_normal((M, K)).astype(np.float16)
    q, s, z = _rand_q(rng, N, K)
    A = (rng.standard_normal((K, r)) * 0.01).astype(np.float16) if r else None
    B = (rng.standard_normal((r, N)) * 0.01).astype(np.float16) if r else None
    Y = oracle.linear_ref(X, q, s, z, A, B)
    Yp = np.array(_py_linear(X.tolist(), q.tolist(), s.tolist(), z.tolist(),
                             None if A is None else A.tolist(), None if B is None else B.tolist()))
    np.testing.assert_allclose(Y, Yp, rtol=1e-12, atol=1e-13)


def test_integer_special_case_is_exact_matmul():
    rng = np.random.default_rng(1)
    M, N, K = 5, 7, 128
    Xi = rng.integers(-3, 4, (M, K))
    Q = rng.integers(0, 8, (N, K)).astype(np.uint8)
    s = np.ones((N, K // 64), np.float16)
    z = np.zeros((N, K // 64), np.float16)
    Y = oracle.linear_ref(Xi.astype(np.float16), Q, s, z)
    np.testing.assert_array_equal(Y, (Xi @ Q.astype(np.int64).T).astype(np.float64))


def test_closed_form_constant_weights():
    # codes 4, s = 0.5, z = 3 -> every weight 0.5; X = 1 -> 64*0.5 = 32 per group;
    # A = 0.25, B = 2 (rank 1) adds (64*0.25)*2 = 32.
    K, N = 64, 3
    q = np.full((N, K), 4, np.uint8)
    s = np.full((N, 1), 0.5, np.float16)
    z = np.full((N, 1), 3.0, np.float16)
    X = np.ones((2, K), np.float16)
    A = np.full((K, 1), 0.25, np.float16)
    B = np.full((1, N), 2.0, np.float16)
    np.testing.assert_array_equal(oracle.linear_ref(X, q, s, z), np.full((2, N), 32.0))
    np.testing.assert_array_equal(oracle.linear_ref(X, q, s, z, A, B), np.full((2, N), 64.0))


def test_compensator_identity_and_special_cases():
    rng = np.random.default_rng(2)
    M, N, K, r = 6, 64, 256, 16
    X = rng.standard_normal((M, K)).astype(np.float16)
    q, s, z = _rand_q(rng, N, K)
    A = (rng.standard_normal((K, r)) * 0.01).astype(np.float16)
    B = (rng.standard_normal((r, N)) * 0.01).astype(np.float16)
    Wd = oracle.dequant_int3(q, s, z)
    Wout = Wd + (A.astype(np.float64) @ B.astype(np.float64)).T   # W_quant + U V
    Y = oracle.linear_ref(X, q, s, z, A, B)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ Wout.T, rtol=1e-12, atol=1e-12)
    # rank 0 and all-zero compensator both reduce to the plain quantized product
    Y0 = oracle.linear_ref(X, q, s, z, A[:, :0], B[:0])
    Yz = oracle.linear_ref(X, q, s, z, np.zeros_like(A), np.zeros_like(B))
    np.testing.assert_array_equal(Y0, Yz)
    np.testing.assert_allclose(Y0, X.astype(np.float64) @ Wd.T, rtol=1e-13)
    # W == 0 (codes 0, s 1, z 0) isolates the low-rank term
    qz = np.zeros_like(q)
    Yl = oracle.linear_ref(X, qz, np.ones_like(s), np.zeros_like(z), A, B)
    np.testing.assert_allclose(Yl, (X.astype(np.float64) @ A) @ B, rtol=1e-13)


def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15


def _tiny_moe(rng, T, H, F, E, S, r):
    experts = []
    for _ in range(E + S):
        e = {}
        for n, (R, K) in {"W1": (F, H), "W3": (F, H), "W2": (H, F)}.items():
            e[n] = (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
        e["A1"] = (rng.standard_normal((H, r)) * 0.01).astype(np.float16)
        e["B1"] = (rng.standard_normal((r, F)) * 0.01).astype(np.float16)
        e["A3"] = (rng.standard_normal((H, r)) * 0.01).astype(np.float16)
        e["B3"] = (rng.standard_normal((r, F)) * 0.01).astype(np.float16)
        e["A2"] = (rng.standard_normal((F, r)) * 0.01).astype(np.float16)
        e["B2"] = (rng.standard_normal((r, H)) * 0.01).astype(np.float16)
        experts.append(oracle.quantize_expert(e))
    X = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return X, logits, experts


def test_single_expert_is_dense_ffn():
    rng = np.random.default_rng(3)
    X, logits, ex = _tiny_moe(rng, 5, 128, 64, 1, 0, 8)
    res = oracle.moe_layer_ref(X, logits, lambda e: ex[e], k=1)
    q = ex[0]
    h1 = oracle.linear_ref(X, *q["W1"], q["A1"], q["B1"])
    h3 = oracle.linear_ref(X, *q["W3"], q["A3"], q["B3"])
    g = h1 / (1 + np.exp(-h1)) * h3
    y = oracle.linear_ref(g, *q["W2"], q["A2"], q["B2"])
    np.testing.assert_allclose(res["out"], y, rtol=1e-13, atol=1e-15)


def test_per_token_loop_and_untouched_experts():
    rng = np.random.default_rng(4)
    T, H, F, E, S, k = 6, 128, 128, 4, 1, 2
    X, logits, ex = _tiny_moe(rng, T, H, F, E, S, 8)
    logits[:, 3] = -100.0          # expert 3 never selected
    res = oracle.moe_layer_ref(X, logits, lambda e: ex[e], k=k, S=S, renormalize=True)
    # per-token loop: each token through each of its experts separately
    rt = res["route"]
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k + S):
            e = int(rt["slot_expert"][t, j])
            _, y = oracle.expert_ffn_ref(X[t:t + 1], ex[e])
            acc += rt["slot_w"][t, j] * y[0]
        np.testing.assert_allclose(res["out"][t], acc, rtol=1e-12, atol=1e-14)
    # replacing the never-routed expert's weights changes nothing
    ex2 = list(ex)
    _, _, other = _tiny_moe(np.random.default_rng(99), T, H, F, E, S, 8)
    ex2[3] = other[3]
    res2 = oracle.moe_layer_ref(X, logits, lambda e: ex2[e], k=k, S=S)
    np.testing.assert_array_equal(res["out"], res2["out"])


def test_combine_identity_k1():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((7, 33))
    np.testing.assert_array_equal(oracle.combine_ref(y, 7, 1), y)
    y2 = rng.standard_normal((7 * 3, 5))
    np.testing.assert_allclose(oracle.combine_ref(y2, 7, 3), y2.reshape(7, 3, 5).sum(1), rtol=1e-15)


def test_out_cols_subset():
    rng = np.random.default_rng(6)
    X, logits, ex = _tiny_moe(rng, 4, 128, 64, 3, 0, 8)
    full = oracle.moe_layer_ref(X, logits, lambda e: ex[e], k=2)
    cols = np.array([0, 5, 77, 127])
    part = oracle.moe_layer_ref(X, logits, lambda e: ex[e], k=2, out_cols=cols)
    np.testing.assert_allclose(part["out"], full["out"][:, cols], rtol=1e-13, atol=1e-15)


def test_metrics():
    assert oracle.rel_fro([1.0, 0.0], [1.0, 0.0]) == 0.0
    assert abs(oracle.rel_fro([1.0, 1.0], [1.0, 0.0]) - 1.0) < 1e-15
    assert oracle.max_abs([1.0, 3.0], [1.5, 3.0]) == 0.5
