"""Pins for the oracle router (oracle/route.py): hand-worked cases, a
rank-counting brute force that never sorts, and the permutation invariants."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "route_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_golden_route(case):
    r = oracle.route_ref(np.array(case["logits"], np.float32), case["k"], case["S"], case["renormalize"])
    np.testing.assert_array_equal(r["ids"], case["ids"])
    np.testing.assert_allclose(r["w"], case["w"], rtol=1e-15)
    np.testing.assert_array_equal(r["sorted_pairs"], case["sorted_pairs"])
    np.testing.assert_array_equal(r["pair_pos"], case["pair_pos"])
    np.testing.assert_array_equal(r["offsets"], case["offsets"])


def _brute(logits, k, S, renorm):
    """Select by counting how many experts beat each expert (no sorting)."""
    T, E = logits.shape
    slots = k + S
    sel = []
    for t in range(T):
        l = [float(v) for v in logits[t]]
        rank = [sum(1 for f in range(E) if l[f] > l[e] or (l[f] == l[e] and f < e)) for e in range(E)]
        ids = [None] * k
        for e in range(E):
            if rank[e] < k:
                ids[rank[e]] = e
        m = max(l)
        den = sum(np.exp(v - m) for v in l)
        p = [np.exp(l[e] - m) / den for e in ids]
        w = [x / sum(p) for x in p] if renorm else p
        sel.append((ids + [E + j for j in range(S)], w + [1.0] * S))
    pairs = []   # (expert, s)
    for t in range(T):
        for j in range(slots):
            pairs.append((sel[t][0][j], t * slots + j))
    n = len(pairs)
    pos = [sum(1 for q in pairs if q < p) for p in pairs]   # position = # smaller keys
    sorted_pairs = [0] * n
    for (e, s), p in zip(pairs, pos):
        sorted_pairs[p] = s
    offsets = [sum(1 for e, _ in pairs if e < x) for x in range(E + S + 1)]
    return sel, sorted_pairs, pos, offsets


@pytest.mark.parametrize("T,E,k,S,renorm,ties", [
    (1, 2, 1, 0, True, False), (3, 4, 2, 0, True, False), (4, 6, 3, 1, False, False),
    (4, 5, 2, 2, True, True), (2, 6, 6, 0, False, True), (4, 3, 1, 0, True, True)])
def test_brute_force(T, E, k, S, renorm, ties):
    rng = np.random.default_rng(T * 100 + E * 10 + k)
    if ties:
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route_ref(logits, k, S, renorm)
    sel, sp, pos, off = _brute(logits, k, S, renorm)
    for t in range(T):
        np.testing.assert_array_equal(r["slot_expert"][t], sel[t][0])
        np.testing.assert_allclose(r["slot_w"][t], sel[t][1], rtol=1e-12)
    np.testing.assert_array_equal(r["sorted_pairs"], sp)
    np.testing.assert_array_equal(r["pair_pos"], pos)
    np.testing.assert_array_equal(r["offsets"], off)


@pytest.mark.parametrize("T,E,k,S,renorm", [(256, 64, 6, 2, False), (1000, 8, 2, 0, True)])
def test_invariants(T, E, k, S, renorm):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route_ref(logits, k, S, renorm)
    slots = k + S
    sp, pp, off = r["sorted_pairs"], r["pair_pos"], r["offsets"]
    assert sorted(sp.tolist()) == list(range(T * slots))
    np.testing.assert_array_equal(pp[sp], np.arange(T * slots))
    assert off[0] == 0 and off[-1] == T * slots and np.all(np.diff(off) >= 0)
    se = r["slot_expert"].reshape(-1)
    for e in range(E + S):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(se[seg] == e)
        assert np.all(np.diff(seg) > 0)          # stable: ascending slot index
    if renorm:
        np.testing.assert_allclose(r["w"].sum(1), 1.0, rtol=1e-12)
    else:
        assert np.all(r["w"].sum(1) <= 1.0 + 1e-12)
    for t in range(T):
        assert len(set(r["ids"][t].tolist())) == k
        assert np.all(np.diff(logits[t, r["ids"][t]]) <= 0)
