"""Pins for the oracle's adaptive rank policy (oracle/rank_policy.py).  The
policy itself has no formula on the pages (parity unpinned); what is pinned
here is its mechanics: kurtosis closed forms and known distributions, the
routing frequency, hand-worked apportionments, and the invariants every
assignment keeps (budget, steps, caps, monotone in the score, the three
directions the pages name)."""
import numpy as np
import pytest

import oracle
from oracle import rank_policy as RP


def test_kurtosis_closed_forms():
    assert RP.kurtosis_ref([-1.0, 1.0]) == pytest.approx(1.0, rel=1e-15)
    # Bernoulli(1/4): (1 - 6 p q) / (p q) + 3 = 7/3
    assert RP.kurtosis_ref([0.0, 0.0, 0.0, 1.0]) == pytest.approx(7.0 / 3.0, rel=1e-14)
    assert RP.kurtosis_ref(np.full(10, 2.5)) == 0.0       # no spread


@pytest.mark.parametrize("kind,expect,tol", [("normal", 3.0, 0.03), ("uniform", 1.8, 0.01),
                                             ("laplace", 6.0, 0.15)])
def test_kurtosis_of_known_distributions(kind, expect, tol):
    rng = np.random.default_rng(1)
    x = {"normal": rng.standard_normal, "uniform": lambda n: rng.uniform(-1, 1, n),
         "laplace": lambda n: rng.laplace(0, 1, n)}[kind](2_000_000)
    assert RP.kurtosis_ref(x) == pytest.approx(expect, abs=tol)


def test_kurtosis_shift_and_scale_invariant():
    x = np.random.default_rng(2).standard_t(5, 10000)
    assert RP.kurtosis_ref(0.02 * x + 3.0) == pytest.approx(RP.kurtosis_ref(x), rel=1e-9)


def test_frequency_from_routing():
    logits = np.random.default_rng(3).standard_normal((64, 8)).astype(np.float32)
    r = oracle.route_ref(logits, 2, 1, True)
    f = RP.expert_frequency_ref(r["offsets"], 64)
    assert f.sum() == pytest.approx(3.0)       # two routed slots + one shared per token
    assert f[-1] == 1.0                        # the shared expert sees every token


@pytest.mark.parametrize("scores,total,r_min,r_max,expect", [
    ([1, 1, 2], 64, 0, 64, [16, 16, 32]),
    ([3, 1], 40, 0, 64, [32, 8]),              # targets 3.75, 1.25 units: remainder to the first
    ([10, 1, 1], 96, 0, 64, [64, 16, 16]),     # cap at 64; the freed units go by remainder, ties low index
    ([1, 0, 0], 24, 8, 64, [8, 8, 8]),         # r_min takes units back from the largest share
    ([0, 0, 0, 0], 64, 0, 64, [16, 16, 16, 16]),
    ([5, 5, 5], 64, 0, 64, [24, 24, 16]),      # 8 units over 3 equal scores: ties to the lower index
])
def test_apportion_hand_worked(scores, total, r_min, r_max, expect):
    assert RP.apportion_ranks_ref(scores, total, r_min, r_max) == expect


@pytest.mark.parametrize("seed", range(6))
def test_apportion_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 40))
    scores = list(rng.exponential(1.0, n))
    r_min, r_max = 8 * int(rng.integers(0, 2)), 64
    total = 8 * int(rng.integers(n * r_min // 8, n * r_max // 8 + 1))
    ranks = RP.apportion_ranks_ref(scores, total, r_min, r_max)
    assert sum(ranks) == total
    assert all(r % 8 == 0 and r_min <= r <= r_max for r in ranks)
    order = np.argsort(scores)
    for a, b in zip(order[:-1], order[1:]):          # scores[a] <= scores[b]
        if scores[a] < scores[b]:
            assert ranks[a] <= ranks[b]
    # scaling the scores by 2 changes nothing (exact in binary)
    assert RP.apportion_ranks_ref([2 * v for v in scores], total, r_min, r_max) == ranks


def test_policy_directions_named_by_the_pages():
    # same kurtosis: dense (always used) above a sparse expert used by 1/4 of
    # tokens -- scores 1 and 1/4, 8 units: targets 6.4 and 1.6, floors 6 and
    # 1, the last unit to the larger remainder (0.6)
    assert RP.rank_policy_ref([3.0, 3.0], [0.25, 0.25], [True, False], 64) == [48, 16]
    # same frequency: heavier tails get more rank
    r = RP.rank_policy_ref([3.0, 6.0], [0.5, 0.5], [False, False], 48)
    assert r[1] > r[0]
    # same kurtosis: the more frequent expert gets more rank
    r = RP.rank_policy_ref([3.0, 3.0], [0.1, 0.4], [False, False], 80)
    assert r[1] > r[0]
