"""Float64 CPU oracle of DSpark's survival-ranked verification budget.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and the bench's CPU leg),
never by the product path. Shares no code with the HIP library.

What it computes (DSpark explainer, "Hardware aware prefix scheduler"; DSpark
guide, "Survival probability" and "Picking the budget"): a confidence head
gives, per request b and block position p, the chance c[b][p] that guess p
survives verification if every earlier guess did. A guess's survival is the
product of the confidences up to it. Every (request, position) slot of the
batch is ranked by survival, highest first; keeping the first n slots costs
one target step over T = R + n tokens (each of the R requests verifies its
last accepted token plus its kept guesses) and is expected to yield R + (sum
of the kept survivals) tokens. The budget is the n that maximises expected
tokens per millisecond, with the step's cost looked up in a table measured
beforehand.

Readings of what the pages leave open (plainest consistent ones):
  * confidences are probabilities: each is clamped into [0, 1] (NaN -> 0)
    before use, so survival never rises along a block and the kept slots of
    every request form a prefix of its block;
  * survival is the product in float64, left to right from position 1;
  * ties in survival rank by request, then position (the lower first);
  * the cost table cost[T] is indexed by the step's token count T = R + n;
    counts the table does not cover (T >= len(cost)) are not candidates;
  * "stop when adding another token hurts" and "pick the n that maximises"
    agree for a convex cost; for a general table the global maximum is
    taken, and among equal maxima the smallest n;
  * the expected tokens use float64 sums in rank order.
"""

from __future__ import annotations

import numpy as np


def survival(conf: np.ndarray) -> np.ndarray:
    """[batch, P] confidences -> [batch, P] float64 survival products."""
    c = np.asarray(conf, dtype=np.float32)
    c = np.where(np.isnan(c), np.float32(0), np.clip(c, np.float32(0), np.float32(1)))
    c = c.astype(np.float64)
    s = np.empty_like(c)
    for b in range(c.shape[0]):
        acc = 1.0
        for p in range(c.shape[1]):
            acc = acc * c[b, p]
            s[b, p] = acc
    return s


def rank_order(s: np.ndarray) -> np.ndarray:
    """Flat slot indices b * P + p, best first: survival desc, then index asc."""
    flat = s.reshape(-1)
    return np.lexsort((np.arange(flat.size), -flat))


def budget(conf: np.ndarray, cost: np.ndarray, diag: dict | None = None) -> dict:
    """The scheduler's decision for one batch: conf [batch, P], cost [n_cost] ms."""
    s = survival(conf)
    R, P = s.shape
    order = rank_order(s)
    sv = s.reshape(-1)[order]
    cost = np.asarray(cost, dtype=np.float32).astype(np.float64)
    best_n, best_f = -1, -np.inf
    S = 0.0
    sums = []
    for n in range(0, R * P + 1):
        if n > 0:
            S = S + sv[n - 1]
        sums.append(S)
        T = R + n
        if T >= cost.size:
            break
        f = (R + S) / cost[T]
        if f > best_f:
            best_f, best_n = f, n
    keep = np.zeros(R, dtype=np.int32)
    if best_n > 0:
        np.add.at(keep, order[:best_n] // P, 1)
    if diag is not None:
        diag["order"] = order
        diag["sorted"] = sv
        diag["sums"] = np.array(sums)
    return dict(keep=keep, n_keep=best_n, survival=s,
                expected_tokens=(R + sums[best_n]) if best_n >= 0 else np.nan,
                objective=best_f)
