"""Pins of the oracle's Rate-Distortion Retention (RDR) assignment.

The pages (SPHERICAL KV abstract) say RDR jointly chooses keep/drop and a
precision tier per token and head under a fixed budget, from estimated
future utility; they give no objective.  This library's reading: rate of a
tier = radius + codes + fp16 value bytes, distortion 2^-(angle bits +
magnitude bits), greedy upgrade steps in decreasing utility-weighted
distortion saving per byte, stopping at the first step that does not fit.
Pins: brute-force optimality at the greedy's own rate (tiny inputs), budget,
monotonicity, recency tie-break, the no-skip stop rule, extremes, and the
large-sample tier fractions predicted analytically for lognormal utility."""
import itertools

import numpy as np
import pytest
from scipy import optimize, stats

from oracle import oracle as O

RATE = {-1: 0, 2: 298, 1: 322, 0: 386}
DIST = {-1: 1.0, 2: 2.0 ** -5, 1: 2.0 ** -8, 0: 2.0 ** -16}


def _assign(util, budget, mask=0b111):
    util = np.asarray(util, np.float32)
    if util.ndim == 1:
        util = util[None, None, :]
    B, H, T = util.shape
    st, tiers = O.rdr_assign(np.full(B, T, np.int32), util, np.asarray(budget, np.int64).reshape(B), mask)
    return st, tiers


def test_step_costs_closed_form():
    st, tiers, dR, c = O.rdr_steps(0b111)
    assert st == O.OK and list(tiers) == [2, 1, 0] and list(dR) == [298, 24, 64]
    assert c[0] == (1 - 2 ** -5) / 298 and c[1] == (2 ** -5 - 2 ** -8) / 24 and c[2] == (2 ** -8 - 2 ** -16) / 64


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_optimal_at_own_rate(seed):
    rng = np.random.default_rng(seed)
    n = 6
    util = np.exp(rng.standard_normal(n)).astype(np.float32)
    if seed == 5:
        util[:] = util[0]                          # all tied
    budget = int(rng.integers(0, 386 * n + 50))
    st, tiers = _assign(util, budget)
    assert st == O.OK
    t = tiers[0, 0]
    Rg = sum(RATE[int(x)] for x in t)
    Dg = sum(float(u) * DIST[int(x)] for u, x in zip(util, t))
    assert Rg <= budget
    for combo in itertools.product((-1, 2, 1, 0), repeat=n):
        R = sum(RATE[x] for x in combo)
        if R <= Rg:
            D = sum(float(u) * DIST[x] for u, x in zip(util, combo))
            assert D >= Dg - 1e-12 * max(1.0, Dg)


def test_budget_and_monotone_in_utility():
    rng = np.random.default_rng(11)
    util = np.exp(rng.standard_normal((2, 4, 500))).astype(np.float32)
    budget = [150000, 400000]
    st, tiers = _assign(util, budget)
    assert st == O.OK
    level = {-1: 0, 2: 1, 1: 2, 0: 3}
    for b in range(2):
        assert sum(RATE[int(x)] for x in tiers[b].ravel()) <= budget[b]
        u = util[b].ravel()
        lv = np.vectorize(level.get)(tiers[b].ravel())
        order = np.argsort(u)
        assert (np.diff(lv[order]) >= 0).all()


def test_stops_at_first_step_that_does_not_fit():
    # order: A's first step (298 B), then B's first step (298 B) which does
    # not fit in 300 B -> the walk stops; A's cheap 24 B upgrade is NOT taken
    st, tiers = _assign([1.0, 0.9], 300)
    assert st == O.OK and list(tiers[0, 0]) == [2, -1]


def test_equal_utilities_keep_most_recent_first():
    # all first steps (298 B) precede all upgrades; the 11th first step does
    # not fit, so the walk stops before any upgrade is reached
    st, tiers = _assign(np.ones(40, np.float32), 298 * 10 + 24 * 3)
    t = tiers[0, 0]
    assert list(t[:30]) == [-1] * 30 and list(t[30:]) == [2] * 10
    # with every first step paid for, upgrades also go to the newest first
    st, tiers = _assign(np.ones(40, np.float32), 298 * 40 + 24 * 3 + 5)
    t = tiers[0, 0]
    assert list(t[:37]) == [2] * 37 and list(t[37:]) == [1] * 3


def test_equal_utilities_heads_ascending_at_same_position():
    util = np.ones((1, 3, 4), np.float32)
    st, tiers = _assign(util, 298 * 2)
    assert st == O.OK
    kept = np.argwhere(tiers[0] >= 0).tolist()
    assert kept == [[0, 3], [1, 3]]


def test_extremes_and_subsets():
    util = np.exp(np.random.default_rng(2).standard_normal(64)).astype(np.float32)
    assert (_assign(util, 386 * 64)[1] == 0).all()
    assert (_assign(util, 0)[1] == -1).all()
    assert (_assign(util, 297)[1] == -1).all()
    st, t = _assign(util, 322 * 10, mask=0b010)          # T4 only: 10 highest utilities kept
    assert st == O.OK
    assert set(np.unique(t)) <= {-1, 1}
    assert sorted(np.argsort(-util)[:10]) == sorted(np.nonzero(t[0, 0] == 1)[0])


def test_invalid_inputs():
    assert _assign([1.0, -1.0], 1000)[0] == O.EINVAL
    assert _assign([1.0, np.nan], 1000)[0] == O.EINVAL
    assert _assign([1.0, np.inf], 1000)[0] == O.EINVAL
    assert _assign([1.0], 1000, mask=0)[0] == O.EINVAL


def test_lognormal_fractions_match_analytic_prediction():
    """Utility w = exp(N(0,1)); budget 35% of dense fp16 (179.2 B per item).
    With threshold lam, step k is taken iff w c_k > lam; the expected bytes
    sum_k dR_k P(w > lam/c_k) = 179.2 fixes lam; the tier fractions follow.
    The greedy on 262144 items must match these within 0.5 percentage points."""
    _, _, dR, c = O.rdr_steps(0b111)
    per_item = 0.35 * 512

    def bytes_at(lam):
        return sum(d * stats.norm.sf(np.log(lam / ck)) for d, ck in zip(dR, c)) - per_item

    lam = optimize.brentq(bytes_at, 1e-9, 10.0)
    p = [stats.norm.sf(np.log(lam / ck)) for ck in c]     # P(at least step k)
    pred = {-1: 1 - p[0], 2: p[0] - p[1], 1: p[1] - p[2], 0: p[2]}
    rng = np.random.default_rng(1002)
    util = np.exp(rng.standard_normal((1, 8, 32768))).astype(np.float32)
    budget = (35 * 32768 * 8 * 512) // 100
    st, tiers = _assign(util, budget)
    assert st == O.OK
    n = tiers.size
    for tau, fr in pred.items():
        assert abs((tiers == tau).sum() / n - fr) < 0.005, (tau, fr)
    used = sum(RATE[t] * int((tiers == t).sum()) for t in RATE)
    assert budget - 298 < used <= budget
