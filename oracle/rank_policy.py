"""Adaptive compensator ranks (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[talk] MiLo Algorithm, "Mixture of Low-Rank Compensators and Adaptive Rank
Selection": the rank is not fixed but chosen per part of the model, from
three observations -- dense, always-activated parts get a higher rank than
sparse experts; more frequently activated experts get a higher rank; weights
with a higher kurtosis (heavier tails, larger quantization error) get a
higher rank.  The pages give no formula.  Reading used here (policy: parity
unpinned, only its mechanics are pinned):

    kurtosis   k_m = E[(w - mu)^4] / E[(w - mu)^2]^2 over all weights of
               matrix m (population moments; 3 for a Gaussian);
    frequency  f_e = pairs routed to expert e / tokens (1 for a dense or
               shared expert, which every token uses);
    score      s_m = f_e(m) * k_m / 3;
    ranks      a budget of `total_rank` rank units is apportioned to the
               matrices in proportion to s_m, in steps of `step`, each rank
               clipped to [r_min, r_max]: the largest-remainder method with
               the caps, ties to the lower matrix index.

The score sum is a left-to-right sum so that any implementation that follows
the same order reaches the same integers.
"""
import math

import numpy as np


def kurtosis_ref(W):
    """Population kurtosis of all entries of W, float64, two passes."""
    w = np.asarray(W, dtype=np.float64).reshape(-1)
    mu = w.mean()
    d = w - mu
    m2 = np.mean(d * d)
    m4 = np.mean(d * d * d * d)
    return float(m4 / (m2 * m2)) if m2 > 0 else 0.0


def expert_frequency_ref(offsets, tokens):
    """Pairs per expert (from the routing offsets) divided by tokens."""
    off = np.asarray(offsets, dtype=np.int64)
    return (off[1:] - off[:-1]).astype(np.float64) / float(tokens)


def rank_scores_ref(kurt, freq, dense):
    """s_m = (1 if dense else f_m) * k_m / 3, float64."""
    return [((1.0 if d else float(f)) * float(k)) / 3.0 for k, f, d in zip(kurt, freq, dense)]


def apportion_ranks_ref(scores, total_rank, r_min, r_max, step=8):
    """Largest-remainder apportionment of total_rank (in units of `step`)
    proportional to scores, each rank in [r_min, r_max] (multiples of step).
    Returns a list of ints."""
    n = len(scores)
    if n == 0:
        return []
    if r_min % step or r_max % step or total_rank % step or r_min > r_max:
        raise ValueError("r_min, r_max, total_rank must be multiples of step with r_min <= r_max")
    units = total_rank // step
    lo, hi = r_min // step, r_max // step
    ssum = 0.0
    for v in scores:
        ssum += float(v)
    if ssum > 0.0:
        target = [units * float(v) / ssum for v in scores]
    else:
        target = [units / n] * n
    u = [min(max(int(math.floor(t)), lo), hi) for t in target]
    left = units - sum(u)
    # hand out (or take back) single units by remainder, ties to the lower index
    while left > 0:
        best = -1
        for i in range(n):
            if u[i] < hi and (best < 0 or target[i] - u[i] > target[best] - u[best]):
                best = i
        if best < 0:
            break
        u[best] += 1
        left -= 1
    while left < 0:
        best = -1
        for i in range(n):
            if u[i] > lo and (best < 0 or target[i] - u[i] < target[best] - u[best]):
                best = i
        if best < 0:
            break
        u[best] -= 1
        left += 1
    return [x * step for x in u]


def rank_policy_ref(kurt, freq, dense, total_rank, r_min=0, r_max=64, step=8):
    return apportion_ranks_ref(rank_scores_ref(kurt, freq, dense), total_rank, r_min, r_max, step)
