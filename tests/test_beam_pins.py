"""Pins of the beam-tree oracle (SparklingTree post, "Future Ideas", item 4):
a re-derivation from an explicit [V][V] bigram table, the limit of unbounded
widths (every prefix, the same set and scores as the SparklingTree oracle's
full tree), the width-1 greedy chain, the even schedule, and structure."""

import numpy as np
import pytest
from scipy.special import log_softmax

from draft_tree_construction_depth_amd import gen
from oracle import beam as BM
from oracle import sparkling as S


def _small(seed, L, V, R, wscale=0.6):
    return gen.sparkling_inputs(seed, batch=1, L=L, V=V, R=R, wscale=wscale)


def _bigram_beam(x, W1, W2t, widths, C):
    """The beam from a full bigram table: children of (depth d, token p) are
    the top-C tokens of row d re-scored by x_d + bigram[p] and log-softmaxed."""
    xf = S.bf16_to_f64(x[0])
    big = S.bf16_to_f64(W1) @ S.bf16_to_f64(W2t).T
    L, V = xf.shape
    cand = [sorted(range(V), key=lambda t: (-xf[d, t], t))[:C] for d in range(L)]
    out = []  # (depth, tokens path, score)
    beam = [(0.0, (), ())]  # (score, ranks, tokens)
    for d in range(L):
        pool = []
        for sc, ranks, toks in beam:
            c = np.array(cand[d])
            s = xf[d, c] + (big[toks[-1], c] if toks else 0.0)
            lp = log_softmax(s)
            order = sorted(range(len(c)), key=lambda j: (-lp[j], c[j]))
            for r, j in enumerate(order):
                pool.append((sc + lp[j], ranks + (r,), toks + (int(c[j]),)))
        pool.sort(key=lambda q: (-q[0], q[1]))
        beam = pool[:widths[d]]
        out += [(d + 1, t, s) for s, _, t in beam]
        if not beam:
            break
    return out


def _paths(o, b=0):
    n = int(o["num_nodes"][b])
    P = {0: ()}
    res = []
    for j in range(n):
        P[j + 1] = P[int(o["parents"][b][j])] + (int(o["tree_tokens"][b][j]),)
        res.append((int(o["depths"][b][j]), P[j + 1], float(o["logq"][b][j])))
    return res


@pytest.mark.parametrize("seed,L,V,C,widths", [
    (0, 3, 6, 3, [2, 3, 4]), (1, 4, 7, 4, [1, 1, 1, 1]), (2, 4, 5, 3, [3, 2, 2, 5]),
    (3, 3, 8, 5, [5, 10, 3]), (4, 2, 9, 6, [0, 4]), (5, 5, 6, 2, [2, 4, 8, 16, 32])])
def test_matches_bigram_table_beam(seed, L, V, C, widths):
    x, W1, W2t = _small(seed, L, V, R=3)
    o = BM.build(x, W1, W2t, widths, C)
    ref = _bigram_beam(x, W1, W2t, widths, C)
    got = _paths(o)
    assert len(got) == len(ref)
    for (d, t, s), (dr, tr, sr) in zip(got, ref):
        assert d == dr and t == tr and abs(s - sr) < 1e-12


def test_unbounded_widths_give_every_prefix():
    """Widths above the number of prefixes: all of them, the same set and
    scores as the SparklingTree oracle's tree with a budget above the count."""
    L, V, C = 3, 5, 3
    x, W1, W2t = _small(7, L, V, R=2)
    o = BM.build(x, W1, W2t, [100] * L, C)
    n = int(o["num_nodes"][0])
    assert n == 3 + 9 + 27
    sp = S.build(x, W1, W2t, 100, C)
    a = {(t): s for _, t, s in _paths(o)}
    b = {(t): s for _, t, s in _paths(sp)}
    assert set(a) == set(b)
    for k in a:
        assert abs(a[k] - b[k]) < 1e-12


def test_width_one_is_the_greedy_chain():
    """w_d = 1: the best child of the best child ... (the spine), which the
    SparklingTree oracle pops first among depth-d prefixes of rank 0 only."""
    x, W1, W2t = _small(8, 6, 12, R=4)
    o = BM.build(x, W1, W2t, [1] * 6, 4)
    rows = S.Rows(S.bf16_to_f64(x[0]), S.bf16_to_f64(W1), S.bf16_to_f64(W2t), 4)
    tok, sc = None, 0.0
    for d in range(6):
        ct, cl = rows.row(d, tok)
        tok, sc = int(ct[0]), sc + float(cl[0])
        assert o["tree_tokens"][0][d] == tok and o["parents"][0][d] == d
        assert abs(o["logq"][0][d] - sc) < 1e-12


@pytest.mark.parametrize("B,L", [(64, 15), (15, 15), (7, 15), (512, 17), (1, 1)])
def test_even_widths(B, L):
    w = BM.even_widths(B, L)
    assert sum(w) == B and max(w) - min(w) <= 1 and w == sorted(w, reverse=True)


def test_structure_at_the_post_setting():
    c = gen.SPARKLING
    x, W1, W2t = gen.sparkling_inputs(0, batch=2, V=4096, R=32)
    widths = BM.even_widths(c["B"], c["L"])
    o = BM.build(x, W1, W2t, widths, c["C"])
    for b in range(2):
        n = int(o["num_nodes"][b])
        assert n == c["B"]
        par, q, dep = o["parents"][b], o["logq"][b], o["depths"][b]
        for j in range(n):
            p = par[j]
            assert 0 <= p <= j
            assert dep[j] == (1 if p == 0 else dep[p - 1] + 1)
            if p:
                assert q[j] <= q[p - 1]
        assert [int((dep[:n] == d + 1).sum()) for d in range(c["L"])] == widths


def test_exact_ties_follow_rank_tuples():
    """Flat rows and a zero head: every candidate of a depth ties, so the
    beam is the lexicographically first rank tuples (worked by hand)."""
    x = np.zeros((1, 2, 6), dtype=np.uint16)
    W = np.zeros((6, 2), dtype=np.uint16)
    o = BM.build(x, W, W, [3, 5], 4)
    assert list(o["tree_tokens"][0]) == [0, 1, 2, 0, 1, 2, 3, 0]
    assert list(o["parents"][0]) == [0, 0, 0, 1, 1, 1, 1, 2]
    np.testing.assert_allclose(o["logq"][0], [-np.log(4)] * 3 + [-2 * np.log(4)] * 5, rtol=1e-15)
