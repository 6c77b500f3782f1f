"""Tree parity: a device-built tree against the oracle's, by excuse class.

TEST INFRASTRUCTURE. Imported by tests/ and by the benchmark's CPU-baseline
leg (which checks the trees of its own run), never by the product path. It
adds no arithmetic of the method beyond re-scoring a given prefix the way the
oracle scores it, and shares nothing with the HIP library.

The rule. Token and parent indices must match the oracle exactly and every
log-probability must lie within 1e-4 of the oracle's value for the same
prefix. Because the device forms row normalisers (and, for the conditioned
trees, log-probabilities) in float32 while the oracle works in float64, two
prefixes whose oracle scores are closer than 1e-5 may come out in the other
order. A mismatch is excused only in these counted classes:

  E1  the node sets differ at the budget boundary: the oracle's B-th and
      (B+1)-th scores are less than 1e-5 apart (a gap of exactly 0 counts
      when the tie is between prefixes of different depths: a prefix and its
      extension tie exactly when a row's other terms underflow in the
      oracle's float64 normaliser); every prefix in one tree and not the
      other, re-scored by the oracle, lies within 1e-5 of the oracle's B-th
      score; no such pair is an exact tie of one depth (that tie is decided by
      the rank-tuple rule on both sides, so a difference there is a bug); and
      the device tree is a valid tree in a valid order (below).
  E2  the node sets agree and the order differs.

Validity, checked for every request whatever its class: the device tree is
prefix-closed with every parent emitted before its children, every node is a
prefix over its rows' top-K tokens (Lemma 1 of the DDTree explainer), no
prefix appears twice, padding past the node count is (-1, -1, -inf, 0), and
every pair of nodes that the device emits in the opposite of the oracle's
order (score desc, then rank tuple lexicographic, a prefix before its
extensions) has oracle scores less than 1e-5 apart and, for DDTree's
canonical score, different depths: prefixes of one depth share Z_d, so their
order follows S, which both sides form exactly. The exception is a prefix
with a step (at it or an ancestor) where the clamp min(score(parent),
S - Z_d) fires or would fire for a normaliser 1e-5 lower, i.e. a token of
probability above 1 - 1e-5: there a float32 normaliser a unit away moves the
clamp, so such pairs follow the cross-depth rule.

Beam-shaped trees (TreeSpark's expansion, the fixed-branching beam) are
compared against the oracle's tree and against the oracle's trees with one
or two near-tie boundary decisions taken the other way (classify_variants).
"""

from __future__ import annotations

import numpy as np

EXCUSE = 1e-5
LOGQ_TOL = 1e-4


# ---------------------------------------------------------------------------
# Scorers: a path of tokens -> (score, rank tuple), or None if the path is
# not a prefix over the rows' candidates.

class DDTreeScorer:
    """The oracle's canonical prefix score (ddtree_oracle.c, readings r3/r4):
    S = x_1[t_1] + ... + x_d[t_d] and Z_d = z_1 + ... + z_d, both float64
    left to right, score = min(score(parent), S - Z_d), root 0. Python floats
    are IEEE doubles, so the sums round exactly as the C oracle's do.

    top_ids [L][K] / top_vals [L][K] (float64) / z [L] are the oracle's own
    stage-1 tables for the request."""

    def __init__(self, top_ids, top_vals, z):
        self.L = top_ids.shape[0]
        self.rank = [{int(t): r for r, t in enumerate(row)} for row in top_ids]
        self.vals = [[float(v) for v in row] for row in top_vals]
        self.Z = []
        acc = 0.0
        for d in range(self.L):
            acc += float(z[d])
            self.Z.append(acc)
        self.cache = {(): (0.0, 0.0, (), False)}  # path -> (S, score, ranks, near clamp)

    def _entry(self, path):
        e = self.cache.get(path)
        if e is not None:
            return e
        d = len(path)
        if d > self.L:
            return None
        par = self._entry(path[:-1])
        if par is None:
            return None
        r = self.rank[d - 1].get(path[-1])
        if r is None:
            return None
        S = par[0] + self.vals[d - 1][r]
        raw = S - self.Z[d - 1]
        sc = par[1] if raw > par[1] else raw
        # the clamp fires here, or would for a normaliser 1e-5 lower
        e = (S, sc, par[2] + (r,), par[3] or raw > par[1] - EXCUSE)
        self.cache[path] = e
        return e

    def __call__(self, path):
        """(score, rank tuple, near clamp) or None."""
        e = self._entry(tuple(path))
        return None if e is None else (e[1], e[2], e[3])


class RowsScorer:
    """Conditioned trees (SparklingTree's rows): score = parent's score + the
    child's log-prob in its row conditioned on the parent's token, float64
    (oracle/sparkling.py, Rows.row). rows is that module's Rows object."""

    def __init__(self, rows):
        self.rows = rows
        self.cache = {(): (0.0, (), False)}

    def __call__(self, path):
        """(score, rank tuple, False) or None."""
        path = tuple(path)
        e = self.cache.get(path)
        if e is not None:
            return e
        d = len(path)
        if d > self.rows.L:
            return None
        par = self(path[:-1])
        if par is None:
            return None
        toks, lps = self.rows.row(d - 1, path[-2] if d > 1 else None)
        hit = np.nonzero(toks == path[-1])[0]
        if hit.size == 0:
            return None
        r = int(hit[0])
        e = (par[0] + float(lps[r]), par[1] + (r,), False)
        self.cache[path] = e
        return e


# ---------------------------------------------------------------------------

def _paths(tok, par, n):
    """Token paths of nodes 1..n (None where the structure is broken)."""
    P = [()]
    for j in range(n):
        p = int(par[j])
        if not 0 <= p <= j:
            return None, f"F:parent {j}->{p}"
        P.append(P[p] + (int(tok[j]),))
    return P[1:], None


def _padding_ok(tok, par, logq, dep, n):
    ok = np.all(tok[n:] == -1) and np.all(par[n:] == -1) and np.all(np.isneginf(logq[n:]))
    if dep is not None:
        ok = ok and np.all(dep[n:] == 0)
    return bool(ok)


def _order_violation(scores, keys, depths, depth_strict, loose=None):
    """First pair emitted in the opposite of the key order whose scores are
    not within EXCUSE (or, with depth_strict, that has equal depths unless one
    of the pair is marked loose)."""
    n = len(keys)
    if n < 2:
        return None
    order = sorted(range(n), key=lambda j: keys[j])
    pos = np.empty(n, np.int64)
    pos[np.asarray(order)] = np.arange(n)
    s = np.asarray(scores, np.float64)
    dd = np.asarray(depths)
    inv = np.triu(pos[:, None] > pos[None, :], 1)  # i emitted before j, j belongs first
    if not inv.any():
        return None
    ok = np.abs(s[:, None] - s[None, :]) < EXCUSE
    if depth_strict:
        lo = np.zeros(n, bool) if loose is None else np.asarray(loose, bool)
        ok &= (dd[:, None] != dd[None, :]) | lo[:, None] | lo[None, :]
    bad = np.argwhere(inv & ~ok)
    if bad.size == 0:
        return None
    i, j = bad[0]
    return f"F:order {int(i)}<{int(j)} ds={s[i] - s[j]:.3g} depths {int(dd[i])},{int(dd[j])}"


def classify_tree(g: dict, o: dict, scorer, B: int, next_score: float, *,
                  depth_strict: bool = True) -> str:
    """One request of a top-B tree. g: the device tree (tree_tokens, parents,
    logq, optional depths, num_nodes as a scalar); o: the oracle's (same keys,
    score64 its float64 scores); next_score: the oracle's (B+1)-th score.
    Returns 'exact', 'E1', 'E2' or 'F:<reason>'."""
    ng, no = int(np.ravel(g["num_nodes"])[0]), int(np.ravel(o["num_nodes"])[0])
    gt, gp, gq = g["tree_tokens"], g["parents"], g["logq"]
    gd = g.get("depths")
    if ng != no:
        return f"F:count {ng} vs {no}"
    if not _padding_ok(gt, gp, gq, gd, ng):
        return "F:padding"
    pg, err = _paths(gt, gp, ng)
    if err:
        return err
    if len(set(pg)) != ng:
        return "F:duplicate prefix"
    sg, kg, cl = [], [], []
    for j, path in enumerate(pg):
        if gd is not None and int(gd[j]) != len(path):
            return f"F:depth {j}"
        r = scorer(path)
        if r is None:
            return f"F:not a prefix over the top-K {path}"
        sg.append(r[0])
        kg.append((-r[0], r[1]))
        cl.append(r[2])
        if abs(float(gq[j]) - r[0]) > LOGQ_TOL:
            return f"F:logq {j} {float(gq[j]):.7g} vs {r[0]:.7g}"
    same = np.array_equal(gt, o["tree_tokens"]) and np.array_equal(gp, o["parents"])
    if same and gd is not None and "depths" in o:
        same = np.array_equal(gd, o["depths"])
    if same:
        return "exact"
    depths = [len(p) for p in pg]
    v = _order_violation(sg, kg, depths, depth_strict, cl)
    if v:
        return v
    po, err = _paths(o["tree_tokens"], o["parents"], no)
    assert err is None
    Sg, So = set(pg), set(po)
    if Sg == So:
        return "E2"
    if no != B:
        return f"F:set below budget diff={len(Sg ^ So)}"
    sB = float(o["score64"][B - 1])
    gap = sB - float(next_score)
    if not 0.0 <= gap < EXCUSE:
        return f"F:set gap={gap:.3g} diff={len(Sg ^ So)}"
    so = {p: float(s) for p, s in zip(po, o["score64"][:no])}
    sgd = dict(zip(pg, sg))
    only_g = [(p, sgd[p]) for p in Sg - So]
    only_o = [(p, so[p]) for p in So - Sg]
    clamped = {p for p in Sg | So if scorer(p)[2]}
    for p, s in only_g + only_o:
        if abs(s - sB) >= EXCUSE:
            return f"F:set member {p} at {s - sB:.3g} from the boundary"
    if depth_strict:
        for p, s in only_g:
            for q, t in only_o:
                if len(p) == len(q) and s == t and p not in clamped and q not in clamped:
                    return f"F:exact same-depth tie decided differently {p} {q}"
    return "E1"


def ddtree_batch_counts(g: dict, o: dict, B: int, idx=None) -> dict:
    """Classify every request of an oracle batch (oracle.build output with its
    tables) against the device batch g; idx maps oracle rows to device rows."""
    counts, fails = {}, []
    for i in range(len(o["num_nodes"])):
        gb = i if idx is None else int(idx[i])
        gi = {k: v[gb] for k, v in g.items() if k in ("tree_tokens", "parents", "logq", "depths",
                                                       "num_nodes")}
        oi = {k: o[k][i] for k in ("tree_tokens", "parents", "depths", "num_nodes", "score64")}
        sc = DDTreeScorer(o["top_ids"][i], o["top_vals"][i], o["z"][i])
        c = classify_tree(gi, oi, sc, B, float(o["next_score"][i]))
        key = "F" if c.startswith("F") else c
        counts[key] = counts.get(key, 0) + 1
        if key == "F":
            fails.append((gb, c))
    return dict(counts=counts, fails=fails)


# ---------------------------------------------------------------------------
# Beam-shaped trees: the oracle's tree or one of its near-tie variants.

def _match(g: dict, ref: dict) -> str | None:
    """'exact', 'same-set' (order differs only between near-ties) or None."""
    ng, no = int(g["num_nodes"]), int(ref["num_nodes"])
    if ng != no:
        return None
    gt, gp, gq = g["tree_tokens"], g["parents"], g["logq"]
    gd = g.get("depths")
    if not _padding_ok(gt, gp, gq, gd, ng):
        return None
    pg, err = _paths(gt, gp, ng)
    if err:
        return None
    po, _ = _paths(ref["tree_tokens"], ref["parents"], no)
    if set(pg) != set(po) or len(set(pg)) != ng:
        return None
    so = {p: float(s) for p, s in zip(po, ref["logq"][:no])}
    for j, p in enumerate(pg):
        if abs(float(gq[j]) - so[p]) > LOGQ_TOL:
            return None
        if gd is not None and int(gd[j]) != len(p):
            return None
    if np.array_equal(gt, ref["tree_tokens"]) and np.array_equal(gp, ref["parents"]):
        return "exact"
    rpos = {p: k for k, p in enumerate(po)}
    scores = [so[p] for p in pg]
    keys = [rpos[p] for p in pg]
    if _order_violation(scores, keys, [0] * ng, False):
        return None
    return "same-set"


def classify_variants(g: dict, variants) -> str:
    """variants: iterable of (label, tree dict) -- the oracle's tree first
    (label None), then its near-tie boundary variants (label = the flipped
    boundaries). Returns 'exact', 'E2', 'E1:<label>' or 'F:...'."""
    for label, ref in variants:
        m = _match(g, ref)
        if m is None:
            continue
        if label is None:
            return "exact" if m == "exact" else "E2"
        return f"E1:{label}"
    return "F:no oracle variant matches"
