"""CPU checks of the parity rule itself (oracle/parity.py).

The rule decides which device trees count as correct, so it is pinned
against trees whose status is known without it:
  * the prefix scorer reproduces the C oracle's float64 scores bit for bit;
  * the oracle's own trees classify as exact;
  * trees the oracle builds after moving every row normaliser by at most
    2e-6 (what the device's float32 normaliser may do) are never failures,
    and on inputs full of near-ties they do reach both excuse classes;
  * planted mistakes -- a far swap, a token outside the top-K, a log-prob off
    by 2e-4, a forward parent, a wrong count, a duplicate, an exact
    same-depth tie decided the other way, a node far from the boundary --
    are failures;
  * beam-shaped trees match their near-tie variants and nothing else.
"""

from __future__ import annotations

import numpy as np
import pytest

from draft_tree_construction_depth_amd import gen
from oracle import oracle as O
from oracle import treespark as T
from oracle.parity import (DDTreeScorer, classify_tree, classify_variants,
                           ddtree_batch_counts)


def _req(o, b=0):
    return {k: o[k][b] for k in ("tree_tokens", "parents", "depths", "num_nodes", "score64")}


def _dev(o, b=0):
    """The oracle's tree in the device's output form (float32 logq)."""
    return {k: np.array(o[k][b]) for k in ("tree_tokens", "parents", "logq", "depths", "num_nodes")}


def _scorer(o, b=0):
    return DDTreeScorer(o["top_ids"][b], o["top_vals"][b], o["z"][b])


@pytest.mark.parametrize("cfg", [1, 2])
def test_scorer_reproduces_oracle_scores(cfg):
    x = gen.make_logits(cfg, 3)
    c = gen.CONFIGS[cfg]
    o = O.build(x, c["dtype"], c["B"])
    sc = _scorer(o)
    P = {0: ()}
    for j in range(int(o["num_nodes"][0])):
        P[j + 1] = P[int(o["parents"][0][j])] + (int(o["tree_tokens"][0][j]),)
        s, ranks, _ = sc(P[j + 1])
        assert s == o["score64"][0][j]  # bit for bit
        assert len(ranks) == o["depths"][0][j]


@pytest.mark.parametrize("cfg", [1, 2])
def test_oracle_tree_is_exact(cfg):
    x = gen.make_logits(cfg, 1)
    c = gen.CONFIGS[cfg]
    o = O.build(x, c["dtype"], c["B"])
    r = ddtree_batch_counts(o, o, c["B"])
    assert r["counts"] == {"exact": 1}


def _near_tie_tables(rng, L, K):
    """Sorted rows on a coarse grid whose top log-prob is within 1e-6 of 0
    (so a prefix and its rank-0 extension nearly tie across depths) or a
    grid value (exact ties of one depth)."""
    vals = np.sort(rng.integers(-8, 1, (L, K)).astype(np.float64) * 0.5, axis=1)[:, ::-1].copy()
    ids = np.tile(np.arange(K, dtype=np.int32), (L, 1))
    z = vals[:, 0] + rng.choice([0.0, 1e-6, 3e-7, 0.5], L)
    return vals, ids, z


def _select_as_build(vals, ids, z, B):
    o = O.select(vals, ids, z, B)
    return {**{k: v[None] if np.ndim(v) else np.array([v]) for k, v in o.items()},
            "top_ids": ids[None], "top_vals": vals[None], "z": z[None]}


def test_perturbed_normaliser_trees_are_never_failures():
    rng = np.random.default_rng(5)
    seen = {}
    for trial in range(600):
        L, K = int(rng.integers(2, 6)), int(rng.integers(2, 7))
        B = int(rng.integers(1, 2 * L * K))
        vals, ids, z = _near_tie_tables(rng, L, K)
        o = _select_as_build(vals, ids, z, B)
        zp = z + rng.uniform(-1e-6, 1e-6, L)
        g = O.select(vals, ids, zp, B)
        dev = {k: g[k] for k in ("tree_tokens", "parents", "logq", "depths")}
        dev["num_nodes"] = int(g["num_nodes"][0])
        c = classify_tree(dev, _req(o), _scorer(o), B, float(o["next_score"][0][0]))
        assert not c.startswith("F"), (trial, c)
        seen[c] = seen.get(c, 0) + 1
    # the excuse classes are reached, not only exact trees
    assert seen.get("E1", 0) > 0 and seen.get("E2", 0) > 0, seen


def _base():
    x = gen.make_logits(1, 2)
    o = O.build(x, gen.DTYPE_F32, 32)
    return o, _req(o), _scorer(o), float(o["next_score"][0])


def _cls(dev, o, req, sc, nxt, B=32):
    return classify_tree(dev, req, sc, B, nxt)


def test_planted_far_swap_fails():
    o, req, sc, nxt = _base()
    dev = _dev(o)
    d = dev["depths"]
    # two depth-1 siblings far apart in score, emitted in the wrong order
    j1 = [j for j in range(32) if d[j] == 1]
    a, b = j1[0], j1[-1]
    assert o["score64"][0][a] - o["score64"][0][b] > 1e-3
    for k in ("tree_tokens", "logq"):
        dev[k][[a, b]] = dev[k][[b, a]]
    # children keep pointing at the right prefix
    par = dev["parents"]
    for j in range(32):
        if par[j] == a + 1:
            par[j] = b + 1
        elif par[j] == b + 1:
            par[j] = a + 1
    c = _cls(dev, o, req, sc, nxt)
    assert c.startswith("F"), c


def test_planted_token_outside_top_k_fails():
    o, req, sc, nxt = _base()
    dev = _dev(o)
    top = set(o["top_ids"][0][int(dev["depths"][5]) - 1].tolist())
    dev["tree_tokens"][5] = next(t for t in range(1024) if t not in top)
    assert _cls(dev, o, req, sc, nxt).startswith("F:not a prefix")


def test_planted_logq_error_fails():
    o, req, sc, nxt = _base()
    dev = _dev(o)
    dev["logq"][7] += np.float32(2e-4)
    assert _cls(dev, o, req, sc, nxt).startswith("F:logq")


def test_planted_structure_errors_fail():
    o, req, sc, nxt = _base()
    dev = _dev(o)
    dev["parents"][3] = 9
    assert _cls(dev, o, req, sc, nxt).startswith("F:parent")
    dev = _dev(o)
    dev["num_nodes"] = 31
    assert _cls(dev, o, req, sc, nxt).startswith("F:count")
    dev = _dev(o)
    dev["tree_tokens"][31] = -1
    dev["logq"][31] = -np.inf
    dev["parents"][31] = -1
    dev["depths"][31] = 0
    assert _cls(dev, o, req, sc, nxt).startswith("F")
    dev = _dev(o)
    j = next(i for i in range(1, 32) if dev["parents"][i] == dev["parents"][0])
    dev["tree_tokens"][j] = dev["tree_tokens"][0]
    assert _cls(dev, o, req, sc, nxt).startswith("F")


def test_planted_far_boundary_member_fails():
    # the last node replaced by a valid prefix far below the boundary
    o, req, sc, nxt = _base()
    dev = _dev(o)
    path = (int(o["top_ids"][0][0][31]),)  # depth 1, rank 31: far down the row
    s, _, _ = sc(path)
    assert o["score64"][0][31] - s > 1e-3
    dev["tree_tokens"][31] = path[0]
    dev["parents"][31] = 0
    dev["depths"][31] = 1
    dev["logq"][31] = np.float32(s)
    assert _cls(dev, o, req, sc, nxt).startswith("F")


def test_planted_same_depth_exact_tie_fails():
    # row 0 holds two equal values; the budget keeps only one of them: the
    # rank-tuple rule keeps rank 1, a tree holding rank 2 instead fails even
    # though the boundary gap is 0
    vals = np.array([[0.0, -1.0, -1.0, -5.0]])
    ids = np.array([[10, 11, 12, 13]], np.int32)
    z = np.array([0.5])
    o = _select_as_build(vals, ids, z, 2)
    assert o["score64"][0][1] == o["next_score"][0]
    dev = _dev(o)
    dev["tree_tokens"][1] = 12
    c = classify_tree(dev, _req(o), _scorer(o), 2, float(o["next_score"][0]))
    assert c.startswith("F:exact same-depth tie"), c


def test_cross_depth_zero_gap_is_e1():
    # the top token of row 1 has log-prob exactly 0 (the other terms of its
    # normaliser underflow in float64), so prefix (0) and (0, 0) tie exactly;
    # a device normaliser a float32 unit higher ranks the extension below a
    # depth-1 sibling at the same score: counted as E1, not a failure
    vals = np.array([[0.0, -2.0, -9.0], [0.0, -900.0, -900.0]])
    ids = np.array([[0, 1, 2], [0, 1, 2]], np.int32)
    z = np.array([np.log1p(np.exp(-2.0) + np.exp(-9.0)), 0.0])
    o = _select_as_build(vals, ids, z, 2)
    g = O.select(vals, ids, z + np.array([0.0, 1e-6]), 2)
    dev = {k: g[k] for k in ("tree_tokens", "parents", "logq", "depths")}
    dev["num_nodes"] = int(g["num_nodes"][0])
    c = classify_tree(dev, _req(o), _scorer(o), 2, float(o["next_score"][0]))
    assert c in ("E1", "exact", "E2"), c


def test_treespark_variants_match_only_near_ties():
    bb, W, E, anc = gen.treespark_inputs(2, batch=1, D=4, V=64, H=64, wscale=0.0)
    diags = []
    o = T.expand(bb, W, E, anc, k=2, F=2, N=8, diags=diags)
    base = {k: v[0] for k, v in o.items()}
    assert classify_variants(base, [(None, base)]) == "exact"
    # a far boundary taken the other way is not an excuse
    far = max(diags[0]["boundaries"], key=lambda bg: bg[1])
    assert far[1] > 1e-3
    jobs = T.near_tie_variants(bb, W, E, int(anc[0]), 0,
                               {"boundaries": [(far[0], 0.0)]}, k=2, F=2, N=8)
    flipped = jobs[0][1]
    assert classify_variants(flipped, [(None, base)]).startswith("F")
    # and it is the variant itself when that boundary is a near-tie
    assert classify_variants(flipped, [(None, base), (jobs[0][0], flipped)]).startswith("E1")
