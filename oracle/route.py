"""Top-k expert routing and the expert-sorted pair list (oracle side).

[talk] Background: an MoE layer replaces the FFN by a group of experts and
activates only a subset of them per token.  The pages give no router formula;
the reading used here is the usual softmax top-k router:

    for each token t:
        ids[t]  = the k experts with the largest logits, ordered by decreasing
                  logit, ties broken towards the lower expert id
        p       = softmax(logits[t])                (float64)
        w[t, j] = p[ids[t, j]] / sum_j p[ids[t, j]]  if renormalize
                  p[ids[t, j]]                       otherwise
    slots j = 0..k-1 are the routed picks; slots j = k..k+S-1 are the shared
    (always-on) experts E + (j - k) with weight 1.

    A (token, slot) pair is identified by its slot index s = t (k + S) + j.
    sorted_pairs lists all s ordered by (expert, s); offsets[e] is the number of
    pairs whose expert is < e (e = 0..E+S); pair_pos is the inverse permutation
    (pair_pos[sorted_pairs[i]] = i).
"""
import numpy as np


def route_ref(logits, k: int, S: int = 0, renormalize: bool = True):
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    slots = k + S
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = logits[t]
        # sort by (-logit, id): lexsort uses the last key as primary
        order = np.lexsort((np.arange(E), -row.astype(np.float64)))
        ids[t] = order[:k]
        x = row.astype(np.float64)
        e = np.exp(x - x.max())
        p = e / e.sum()
        sel = p[ids[t]]
        w[t] = sel / sel.sum() if renormalize else sel
    slot_expert = np.zeros((T, slots), dtype=np.int32)
    slot_w = np.zeros((T, slots), dtype=np.float64)
    slot_expert[:, :k] = ids
    slot_w[:, :k] = w
    for j in range(S):
        slot_expert[:, k + j] = E + j
        slot_w[:, k + j] = 1.0
    flat_e = slot_expert.reshape(-1)
    s_idx = np.arange(T * slots)
    sorted_pairs = np.lexsort((s_idx, flat_e)).astype(np.int32)
    counts = np.bincount(flat_e, minlength=E + S)
    offsets = np.zeros(E + S + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_pos = np.empty(T * slots, dtype=np.int32)
    pair_pos[sorted_pairs] = np.arange(T * slots, dtype=np.int32)
    return {
        "ids": ids,
        "w": w,
        "slot_expert": slot_expert,
        "slot_w": slot_w,
        "sorted_pairs": sorted_pairs,
        "pair_pos": pair_pos,
        "offsets": offsets,
    }
