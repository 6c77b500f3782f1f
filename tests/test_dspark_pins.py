"""Pins of the DSpark budget oracle (DSpark explainer, "Hardware aware prefix
scheduler"; DSpark guide, "Survival probability", "Picking the budget"):
the pages' worked survival examples, brute force over every per-request
prefix choice, the chain formula for identical confidences, the marginal
optimality condition of a linear cost, and the explainer's greedy stop rule."""

import itertools
import os

import numpy as np
import pytest

from oracle import dspark as D

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "dspark_survival.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            kind, *vals = line.split()
            rows.append((kind, [float(v) for v in vals]))
    return rows


def test_golden_survival_examples():
    for kind, vals in _golden():
        if kind == "survival":
            # confidences that reproduce the printed prefix survivals
            conf = [vals[0]] + [vals[i] / vals[i - 1] for i in range(1, len(vals))]
            s = D.survival(np.array([conf], dtype=np.float32))[0]
            np.testing.assert_allclose(s, vals, atol=1e-6)
            assert np.all(np.diff(s) <= 0)
        else:
            s = D.survival(np.array([vals[:-1]], dtype=np.float32))[0]
            assert round(s[-1], 2) == vals[-1]


def _random_case(rng, R, P):
    conf = rng.uniform(0.05, 1.0, (R, P)).astype(np.float32)
    c0, c1 = rng.uniform(5, 30), rng.uniform(0.05, 2.0)
    cost = (c0 + c1 * np.arange(R * P + R + 1)).astype(np.float32)
    return conf, cost


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_over_prefix_choices(seed):
    """Every choice of a kept prefix length per request: the oracle's
    objective is the maximum, and its keep vector reaches it."""
    rng = np.random.default_rng(seed)
    R, P = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    conf, cost = _random_case(rng, R, P)
    if seed % 3 == 0:  # a non-convex measured table (steps)
        cost = (20 + 3 * (np.arange(cost.size) // 3) + rng.uniform(0, 1, cost.size)).astype(np.float32)
    o = D.budget(conf, cost)
    s = conf.astype(np.float64)
    s = np.cumprod(np.clip(s, 0, 1), axis=1)  # exact enough for comparison at 1e-12
    best = -np.inf
    for ks in itertools.product(range(P + 1), repeat=R):
        n = sum(ks)
        if R + n >= cost.size:
            continue
        tok = R + sum(s[b, :k].sum() for b, k in enumerate(ks))
        best = max(best, tok / float(cost[R + n]))
    assert abs(o["objective"] - best) <= 1e-12 * best
    tok = R + sum(s[b, :k].sum() for b, k in enumerate(o["keep"]))
    assert abs(tok / float(cost[R + o["keep"].sum()]) - best) <= 1e-12 * best
    assert o["keep"].sum() == o["n_keep"]


@pytest.mark.parametrize("a,g", [(0.5, 4), (0.5, 8), (0.8, 4), (0.3, 6)])
def test_chain_formula_for_identical_confidences(a, g):
    """Every request guesses with confidence a at every position; with the
    first g positions of every request kept, expected tokens per request are
    the chain value (1 - a^(g+1)) / (1 - a) (DSpark guide). A cost table
    that is flat up to R*(g+1) tokens and then jumps forces that budget."""
    R, P = 5, 10
    conf = np.full((R, P), a, dtype=np.float32)
    T = np.arange(R * P + R + 1)
    cost = np.where(T <= R * (g + 1), 10.0, 1e6).astype(np.float32)
    d = {}
    o = D.budget(conf, cost, diag=d)
    assert o["n_keep"] == R * g
    assert (o["keep"] == g).all()
    af = float(np.float32(a))
    np.testing.assert_allclose(o["expected_tokens"] / R, (1 - af ** (g + 1)) / (1 - af), rtol=1e-12)


def test_golden_chain_values_through_the_budget():
    """The chain values printed on the DSpark guide, reproduced as the
    budget's expected tokens per request."""
    for line in open(os.path.join(GOLDEN, "chain_tokens_per_pass.txt")):
        if line.startswith("#") or not line.strip():
            continue
        a, g, val, dec = line.split()
        a, g, dec = float(a), int(g), int(dec)
        R = 3
        conf = np.full((R, 12), a, dtype=np.float32)
        T = np.arange(R * 13 + 1)
        cost = np.where(T <= R * (g + 1), 1.0, 1e9).astype(np.float32)
        o = D.budget(conf, cost)
        assert round(o["expected_tokens"] / R, dec) == float(val)


@pytest.mark.parametrize("seed", range(8))
def test_marginal_condition_of_a_linear_cost(seed):
    """cost = c0 + c1 T: adding the next slot (survival s) raises tokens per
    ms iff s > c1 * f(n). At the optimum every kept slot passed that test
    and the first dropped one fails it."""
    rng = np.random.default_rng(100 + seed)
    R, P = int(rng.integers(8, 64)), int(rng.integers(3, 12))
    conf, cost = _random_case(rng, R, P)
    c1 = float(cost[1]) - float(cost[0])
    d = {}
    o = D.budget(conf, cost, diag=d)
    n, sv, sums = o["n_keep"], d["sorted"], d["sums"]
    f = lambda k: (R + sums[k]) / float(cost[R + k])
    for k in range(n):  # each kept slot improved on the state before it
        assert sv[k] >= c1 * f(k) * (1 - 1e-6)
    if n < R * P:
        assert sv[n] <= c1 * f(n) * (1 + 1e-6)


@pytest.mark.parametrize("seed", range(8))
def test_greedy_stop_rule_agrees_for_a_convex_cost(seed):
    """The explainer's rule (add slots in order, stop when throughput would
    drop) and the guide's (take the maximising count) pick the same budget
    when the cost is linear."""
    rng = np.random.default_rng(200 + seed)
    R, P = int(rng.integers(4, 40)), int(rng.integers(2, 10))
    conf, cost = _random_case(rng, R, P)
    s = D.survival(conf).reshape(-1)
    sv = np.sort(s)[::-1]
    n, tok = 0, float(R)
    while n < sv.size and (tok + sv[n]) / cost[R + n + 1] > tok / cost[R + n]:
        tok += sv[n]
        n += 1
    assert D.budget(conf, cost)["n_keep"] == n


def test_kept_slots_are_prefixes_and_ties_by_request():
    conf = np.array([[0.9, 1.0, 0.5], [0.9, 1.0, 0.5], [1.5, np.nan, 0.2]], dtype=np.float32)
    s = D.survival(conf)
    assert s[2, 0] == 1.0 and s[2, 1] == 0.0  # clamped; NaN counts as 0
    o = D.budget(conf, np.array([1.0] * 6 + [1.6] + [100.0] * 10, dtype=np.float32))
    # slots: (2,0)=1.0 first, then the four 0.9s by request/position
    order = D.rank_order(s)
    assert list(order[:5]) == [6, 0, 1, 3, 4]
    for b in range(3):
        k = o["keep"][b]
        kept = [b * 3 + p for p in range(3)]
        ranks = {int(x): i for i, x in enumerate(order)}
        assert all(ranks[kept[p]] < o["n_keep"] for p in range(k))
        assert all(ranks[kept[p]] >= o["n_keep"] for p in range(k, 3))


def test_no_guess_worth_checking():
    """A steep cost per token: only the guaranteed tokens."""
    conf = np.full((4, 5), 0.3, dtype=np.float32)
    cost = (10 + 100 * np.arange(30)).astype(np.float32)
    o = D.budget(conf, cost)
    assert o["n_keep"] == 0 and (o["keep"] == 0).all() and o["expected_tokens"] == 4.0


def test_equal_objectives_take_the_smallest_budget():
    """Slots of survival 0 under a flat cost leave tokens per ms unchanged:
    the smallest maximising count is kept."""
    conf = np.array([[0.8, 0.0, 0.5], [0.6, 0.5, 0.0]], dtype=np.float32)
    o = D.budget(conf, np.full(10, 7.0, dtype=np.float32))
    assert o["n_keep"] == 3 and list(o["keep"]) == [1, 2]
