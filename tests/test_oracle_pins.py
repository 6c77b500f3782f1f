"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one part of the oracle against something the pages or the
mathematics fix: closed forms, library routines, exhaustive enumeration,
a textbook tree-knapsack optimum, a Monte Carlo estimate of Proposition 1,
and the chain values printed on the DSpark guide page.
"""

import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax, logsumexp

from draft_tree_construction_depth_amd import gen
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32, BF16 = gen.DTYPE_F32, gen.DTYPE_BF16


# ----------------------------------------------------------------------------
# Stage 1: normaliser and ranking
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("c,V", [(1.5, 1024), (-3.25, 151936), (0.0, 7)])
def test_lse_constant_row_closed_form(c, V):
    row = np.full(V, c, np.float32)
    assert O.row_lse(row, F32) == pytest.approx(c + math.log(V), rel=0, abs=1e-12)
    bits = gen.f32_to_bf16_bits(row)
    assert O.row_lse(bits, BF16) == pytest.approx(c + math.log(V), rel=0, abs=1e-12)


def test_lse_dominant_token_is_exact():
    row = np.zeros(5000, np.float32)
    row[1234] = 800.0
    assert O.row_lse(row, F32) == 800.0


@pytest.mark.parametrize("seed", range(4))
def test_lse_matches_independent_formulations(seed):
    rng = np.random.default_rng(seed)
    for V in (3, 1024, 20000):
        x = (rng.uniform(0.5, 8) * rng.standard_normal(V)).astype(np.float32)
        xd = x.astype(np.float64)
        m = xd.max()
        ref = m + math.log(math.fsum(np.exp(xd - m)))
        z = O.row_lse(x, F32)
        assert abs(z - ref) <= 1e-12 * max(1.0, abs(ref))
        assert abs(z - logsumexp(xd)) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("seed", range(6))
def test_rank_matches_numpy_lexsort_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(5, 3000))
    # Integer-valued logits force many exact ties; include both zeros.
    x = rng.integers(-4, 5, V).astype(np.float32)
    x[rng.integers(0, V, 5)] = -0.0
    ids_all = np.arange(V)
    xd = x.astype(np.float64) + 0.0  # -0 -> +0 for the reference
    order = np.lexsort((ids_all, -xd))
    K = int(rng.integers(1, V + 1))
    ids, vals = O.row_rank(x, F32, K)
    np.testing.assert_array_equal(ids, order[:K])
    np.testing.assert_array_equal(vals, xd[order[:K]])
    bits = gen.f32_to_bf16_bits(x)
    ids_b, _ = O.row_rank(bits, BF16, K)
    np.testing.assert_array_equal(ids_b, order[:K])


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * rng.uniform(0.1, 50, 100000)).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gen.f32_to_bf16_bits(x), ref)


# ----------------------------------------------------------------------------
# Stage 2: selection, against exhaustive enumeration over the full vocabulary
# ----------------------------------------------------------------------------

def brute_force_tree(x: np.ndarray, z: np.ndarray, B: int):
    """All prefixes over the FULL vocabulary, sorted by (-score, rank tuple).

    Ranks come from numpy's lexsort (value desc, id asc). The score is the
    canonical one: left-to-right float64 sums S and Z, raw = S - Z_d, clamped
    to the parent's score. Returns the first B prefixes as dicts.
    """
    L, V = x.shape
    x = x + 0.0
    tok_of_rank = [np.lexsort((np.arange(V), -x[i])) for i in range(L)]
    Z = []
    acc = 0.0
    for i in range(L):
        acc = acc + float(z[i])
        Z.append(acc)
    items = {}
    for d in range(1, L + 1):
        for ranks in itertools.product(range(V), repeat=d):
            if d == 1:
                S_par, sc_par = 0.0, 0.0
            else:
                S_par, sc_par = items[ranks[:-1]]["S"], items[ranks[:-1]]["score"]
            S = S_par + float(x[d - 1, tok_of_rank[d - 1][ranks[-1]]])
            raw = S - Z[d - 1]
            items[ranks] = dict(S=S, score=min(sc_par, raw), ranks=ranks,
                                token=int(tok_of_rank[d - 1][ranks[-1]]))
    order = sorted(items.values(), key=lambda it: (-it["score"], it["ranks"]))
    return order[:B], items


def _compare_with_brute(x32: np.ndarray, B: int):
    L, V = x32.shape
    o = O.build(x32[None], F32, B)
    z = o["z"][0]
    top, _ = brute_force_tree(x32.astype(np.float64), z, B)
    n = int(o["num_nodes"][0])
    assert n == len(top)
    index = {it["ranks"]: j + 1 for j, it in enumerate(top)}
    for j, it in enumerate(top):
        assert o["tree_tokens"][0, j] == it["token"]
        assert o["depths"][0, j] == len(it["ranks"])
        assert o["parents"][0, j] == (0 if len(it["ranks"]) == 1 else index[it["ranks"][:-1]])
        assert o["score64"][0, j] == it["score"]  # bit for bit
    assert np.all(o["tree_tokens"][0, n:] == -1)
    assert np.all(o["parents"][0, n:] == -1)
    assert np.all(np.isneginf(o["logq"][0, n:]))
    return o, top


@pytest.mark.parametrize("seed", range(12))
def test_heap_equals_exhaustive_enumeration_gaussian(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 7))
    L = int(rng.integers(1, 6 if V <= 4 else 5))
    B = int(rng.integers(1, 40))
    x = (rng.uniform(0.3, 3) * rng.standard_normal((L, V))).astype(np.float32)
    _compare_with_brute(x, B)


@pytest.mark.parametrize("seed", range(12))
def test_heap_equals_exhaustive_enumeration_with_ties(seed):
    # Integer logits: many exact ties inside rows and between prefixes, so the
    # lexicographic tie rule is exercised; B both below and above V (Lemma 1).
    rng = np.random.default_rng(1000 + seed)
    V = int(rng.integers(2, 6))
    L = int(rng.integers(1, 5))
    B = int(rng.integers(1, 60))
    x = rng.integers(-2, 3, (L, V)).astype(np.float32)
    _compare_with_brute(x, B)


def test_degenerate_constant_rows_and_budget_beyond_prefix_count():
    x = np.zeros((3, 2), np.float32)  # 2 + 4 + 8 = 14 prefixes, all equal per depth
    o, top = _compare_with_brute(x, 20)
    assert int(o["num_nodes"][0]) == 14
    # equal scores per depth: order is depth by depth, lexicographic inside
    assert list(o["depths"][0, :14]) == [1, 1] + [2] * 4 + [3] * 8


def test_one_hot_rows_clamp_matches_enumeration():
    # Rows whose normaliser equals their maximum to float64 precision.
    x = np.full((4, 3), -1000.0, np.float32)
    x[:, 0] = [5.0, 17.0, 3.0, 2.0 ** -20]
    _compare_with_brute(x, 10)


def test_top_b_is_prefix_closed_and_rank_closed():
    # Proposition 2 (DDTree explainer, section 3): the B most probable
    # prefixes form a valid tree.
    for seed in range(20):
        rng = np.random.default_rng(50 + seed)
        V, L = 4, 4
        x = (rng.uniform(0.3, 3) * rng.standard_normal((L, V))).astype(np.float32)
        z = np.array([O.row_lse(x[i], F32) for i in range(L)])
        B = int(rng.integers(1, 80))
        top, _ = brute_force_tree(x.astype(np.float64), z, B)
        chosen = {it["ranks"] for it in top}
        for r in chosen:
            if len(r) > 1:
                assert r[:-1] in chosen
            if r[-1] > 0:
                assert r[:-1] + (r[-1] - 1,) in chosen


def _knapsack_best(q_of, V, L, B):
    """Max sum of prefix probabilities over rooted subtrees of the full trie
    with at most B non-root nodes (textbook tree knapsack)."""
    def best(prefix):
        # returns array f[k] = best total using exactly <= k nodes in the subtree
        # of `prefix` (prefix itself counted, except for the root).
        d = len(prefix)
        self_q = 0.0 if d == 0 else q_of[prefix]
        cap = B + (1 if d == 0 else 0)
        f = np.full(cap + 1, -np.inf)
        f[0] = 0.0
        if d == 0:
            acc = np.full(B + 1, -np.inf)
            acc[0] = 0.0
        else:
            acc = np.full(B, -np.inf)  # budget left for children
            acc[0] = 0.0
        if d < L:
            for v in range(V):
                g = best(prefix + (v,))
                new = np.full_like(acc, -np.inf)
                for a in range(len(acc)):
                    if acc[a] == -np.inf:
                        continue
                    for k in range(len(g)):
                        if a + k < len(acc) and g[k] > -np.inf:
                            new[a + k] = max(new[a + k], acc[a] + g[k])
                acc = np.maximum(acc, new)
        if d == 0:
            return acc
        f = np.full(B + 1, -np.inf)
        f[0] = 0.0
        for a in range(len(acc)):
            if acc[a] > -np.inf:
                f[a + 1] = max(f[a + 1], self_q + acc[a])
        return f

    f = best(())
    return float(np.max(f[np.isfinite(f)]))


@pytest.mark.parametrize("seed", range(6))
def test_heap_tree_is_optimal_tree_knapsack(seed):
    # Proposition 2: the top-B tree maximises the expected acceptance
    # sum_u q(u) among prefix-closed trees with at most B nodes. q is
    # computed here independently from scipy's log_softmax.
    rng = np.random.default_rng(300 + seed)
    V, L = 4, 4
    x = (rng.uniform(0.3, 3) * rng.standard_normal((L, V))).astype(np.float32)
    B = int(rng.integers(1, 25))
    lp = log_softmax(x.astype(np.float64), axis=1)
    q_of = {}
    for d in range(1, L + 1):
        for toks in itertools.product(range(V), repeat=d):
            q_of[toks] = math.exp(sum(lp[i, t] for i, t in enumerate(toks)))
    o = O.build(x[None], F32, B)
    n = int(o["num_nodes"][0])
    # tree tokens along each node's path
    paths = {}
    for j in range(n):
        p = o["parents"][0, j]
        paths[j + 1] = (paths[p] if p else ()) + (int(o["tree_tokens"][0, j]),)
    heap_sum = sum(q_of[paths[j + 1]] for j in range(n))
    assert heap_sum == pytest.approx(_knapsack_best(q_of, V, L, B), rel=1e-12, abs=1e-15)


def test_logq_is_sum_of_log_softmax():
    x = gen.make_logits(1, 3)
    o = O.build(x, F32, 32)
    lp = log_softmax(x[0].astype(np.float64), axis=1)
    n = int(o["num_nodes"][0])
    paths = {}
    for j in range(n):
        p = o["parents"][0, j]
        paths[j + 1] = (paths[p] if p else ()) + (int(o["tree_tokens"][0, j]),)
        ref = sum(lp[i, t] for i, t in enumerate(paths[j + 1]))
        assert abs(o["score64"][0, j] - ref) < 1e-12
        assert abs(float(o["logq"][0, j]) - ref) < 1e-6


def test_heap_size_is_linear_in_budget():
    # O(B) heap (DDTree explainer, section 4): each pop pushes at most two.
    x = gen.make_logits(3, 1, batch=2, V=4096)
    for B in (16, 64, 128):
        o = O.build(x, BF16, B)
        assert np.all(o["max_heap"] <= 2 * B + 1)


def test_clamp_never_fires_on_generated_workloads():
    x1 = gen.make_logits(1, 0)
    assert O.build(x1, F32, 32)["clamps"].sum() == 0
    x3 = gen.make_logits(3, 0, batch=2)
    assert O.build(x3, BF16, 128, threads=2)["clamps"].sum() == 0


# ----------------------------------------------------------------------------
# Stage 3: mask
# ----------------------------------------------------------------------------

def _pointer_chase_mask(parents, n, B):
    W = (B + 1 + 63) // 64
    m = np.zeros((B + 1, W), np.uint64)
    for i in range(n + 1):
        u = i
        while True:
            m[i, u // 64] |= np.uint64(1) << np.uint64(u % 64)
            if u == 0:
                break
            u = int(parents[u - 1])
    return m


@pytest.mark.parametrize("cfg,seed,B", [(1, 0, 32), (1, 1, 32), (3, 0, 128), (3, 1, 200)])
def test_mask_matches_pointer_chase_and_invariants(cfg, seed, B):
    c = gen.CONFIGS[cfg]
    x = gen.make_logits(cfg, seed, batch=2, V=min(c["V"], 8192))
    o = O.build(x, c["dtype"], B)
    m = O.mask(o["parents"], o["num_nodes"], B)
    for b in range(2):
        n = int(o["num_nodes"][b])
        np.testing.assert_array_equal(m[b], _pointer_chase_mask(o["parents"][b], n, B))
        for i in range(B + 1):
            bits = [j for j in range(B + 1) if (int(m[b, i, j // 64]) >> (j % 64)) & 1]
            if i > n:
                assert bits == []
                continue
            depth = 0 if i == 0 else int(o["depths"][b, i - 1])
            assert len(bits) == depth + 1
            assert bits[0] == 0 and bits[-1] == i


# ----------------------------------------------------------------------------
# Stage 4: walk, Proposition 1 and the chain closed form
# ----------------------------------------------------------------------------

def _walk_by_definition(tok, par, n, tgt, L):
    """Deepest node whose every edge p->v has target[p] == token(v)."""
    best = (0, [])
    for u in range(1, n + 1):
        path = []
        v = u
        while v:
            path.append(v)
            v = int(par[v - 1])
        path.reverse()
        ok, prev = True, 0
        for v in path:
            if tgt[prev] != tok[v - 1]:
                ok = False
                break
            prev = v
        if ok and len(path) > len(best[1]):
            best = (u, path)
    return best


@pytest.mark.parametrize("seed", range(5))
def test_walk_matches_definition(seed):
    rng = np.random.default_rng(seed)
    x = gen.make_logits(1, seed)
    o = O.build(x, F32, 32)
    # targets: mostly the tree's own tokens so that paths are long
    n = int(o["num_nodes"][0])
    tgt = rng.integers(0, 1024, 33).astype(np.int32)
    for i in range(33):
        kids = [j + 1 for j in range(n) if o["parents"][0, j] == i]
        if kids and rng.random() < 0.8:
            tgt[i] = o["tree_tokens"][0, rng.choice(kids) - 1]
    acc, alen, nxt = O.accept(o["tree_tokens"], o["parents"], o["num_nodes"], tgt[None], 15)
    u, path = _walk_by_definition(o["tree_tokens"][0], o["parents"][0], n, tgt, 15)
    assert int(alen[0]) == len(path)
    assert list(acc[0, :len(path)]) == path
    assert np.all(acc[0, len(path):] == -1)
    assert int(nxt[0]) == int(tgt[u])


def _mc_accept(x32, o, B, L, N, rng):
    """Draw N sequences Y ~ Q (inverse CDF of scipy softmax) and walk the tree."""
    p = np.exp(log_softmax(x32.astype(np.float64), axis=1))
    V = p.shape[1]
    Y = np.empty((N, L + 1), np.int64)
    for d in range(L):
        cdf = np.cumsum(p[d])
        Y[:, d] = np.minimum(np.searchsorted(cdf, rng.random(N) * cdf[-1], side="right"), V - 1)
    Y[:, L] = 0
    dep = np.concatenate([[0], o["depths"][0].astype(np.int64)])
    n = int(o["num_nodes"][0])
    tgt = Y[:, np.minimum(dep, L)].astype(np.int32)
    tgt[:, n + 1:] = 0
    rep = lambda a: np.repeat(a, N, axis=0)
    _, alen, _ = O.accept(rep(o["tree_tokens"]), rep(o["parents"]), rep(o["num_nodes"]), tgt, L)
    return alen


@pytest.mark.parametrize("seed", range(3))
def test_prop1_expected_acceptance_is_sum_of_prefix_probabilities(seed):
    # Proposition 1 (DDTree explainer, section 3), by Monte Carlo.
    rng = np.random.default_rng(seed)
    L, V, B = 6, 12, 24
    x = (rng.uniform(0.5, 2.5) * rng.standard_normal((L, V))).astype(np.float32)
    o = O.build(x[None], F32, B)
    n = int(o["num_nodes"][0])
    expected = float(np.exp(o["score64"][0, :n]).sum())
    alen = _mc_accept(x, o, B, L, 200000, rng)
    se = alen.std() / math.sqrt(len(alen))
    assert abs(alen.mean() - expected) < 5 * se


def _chain_rows(a, V, g):
    row = np.full(V, math.log((1 - a) / (V - 1)), np.float64)
    row[0] = math.log(a)
    return np.tile(row.astype(np.float32), (g, 1))


def _golden_chain():
    rows = []
    with open(os.path.join(GOLDEN, "chain_tokens_per_pass.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, g, val, dec = line.split()
                rows.append((float(a), int(g), float(val), int(dec)))
    return rows


@pytest.mark.parametrize("row", _golden_chain())
def test_chain_closed_form_printed_values(row):
    # With one token of probability a per position and the rest spread so thin
    # that no sibling beats the chain, the budget-g tree is the chain and
    # 1 + sum q(u) is the pages' tokens-per-pass formula.
    a, g, printed, dec = row
    V = 10 if (a, g) != (0.5, 8) else 256
    x = _chain_rows(a, V, g)
    o = O.build(x[None], F32, g)
    assert list(o["depths"][0]) == list(range(1, g + 1))
    assert list(o["parents"][0]) == list(range(0, g))
    assert np.all(o["tree_tokens"][0] == 0)
    tokens = 1.0 + float(np.exp(o["score64"][0]).sum())
    closed = (1 - a ** (g + 1)) / (1 - a)
    assert tokens == pytest.approx(closed, abs=2e-6)
    assert round(tokens, dec) == pytest.approx(printed, abs=1e-9)
    # Monte Carlo through the walk: committed tokens = accept_len + 1
    alen = _mc_accept(x, o, g, g, 100000, np.random.default_rng(g))
    se = alen.std() / math.sqrt(len(alen))
    assert abs(alen.mean() + 1 - closed) < 5 * se
