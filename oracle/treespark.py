"""Float64 CPU oracle of TreeSpark's parent-conditioned tree expansion.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path. Shares no code with
the HIP library.

What it computes (TreeSpark README, item 1 "Parent-Conditioned Tree Drafting
from One Backbone Pass", and item 2's candidate policy): one backbone pass
gives vocabulary logits l_d for every draft depth d; a first-order Markov
head specialises depth d to a parent token t_u,

    z_d(u) = l_d + W . e(t_u),      e(t) = E[t] (embedding row of t),

trees expand with branching factor k per parent over D depths, the frontier
is pruned by joint path score, and a global top-N packing keeps N non-root
nodes (k = 4, D = 7, N = 32: at most 100 candidates, 33 positions with the
anchor).

Readings of what the README leaves open (the plainest consistent ones):
  * the depth-1 parent is the anchor (root) token; the root scores 0;
  * a child's path score is its parent's plus its log-softmax log-prob,
    score(v) = score(u) + z_d(u)[t] - logsumexp(z_d(u));
  * per-parent top-k by (z desc, token id asc);
  * the frontier for depth d+1 is the best F of depth d's children, and the
    packing the best N of all candidates, both by (score desc, rank tuple
    lexicographic asc), where a node's rank tuple is its parent's plus the
    child's position j in the parent's top-k; F = k;
  * packed node j+1 is the j-th of that order; its parent is the parent's
    packed position (0 = anchor). Ancestors come first: a child's score is
    at most its parent's and its rank tuple extends the parent's.
Arithmetic: float64 throughout; z by numpy matmul of the exactly widened
bf16 operands, logsumexp by scipy.

Near-tie variants. Every decision boundary of the expansion -- a parent's
k-th/(k+1)-th child, a depth's F-th/(F+1)-th child (the frontier cut), the
N-th/(N+1)-th candidate (the packing cut) -- is recorded with its gap. A
variant takes a given set of boundaries the other way (the (k+1)-th child,
(F+1)-th child or (N+1)-th candidate in place of the k-th, F-th or N-th) and
expands on from there with the same arithmetic; the parity check compares a
device tree with the variants of boundaries closer than 1e-5, the only
places where float32 device arithmetic may decide otherwise.
"""

from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def parent_logits(l_d: np.ndarray, W: np.ndarray, E_rows: np.ndarray) -> np.ndarray:
    """z for each parent: l_d [V] + W [V, H] @ E_rows[m] (rows [M, H]) -> [M, V], float64."""
    return l_d[None, :] + (W @ E_rows.T).T


def top_k(z: np.ndarray, k: int):
    """(ids, values) of the k largest entries of z by (value desc, id asc)."""
    order = np.lexsort((np.arange(z.shape[0]), -z))
    ids = order[:k]
    return ids, z[ids]


def _order_key(node):
    return (-node["score"], node["ranks"])


class _Job:
    """One request's expansion state (optionally with boundaries flipped)."""

    def __init__(self, bb, anchor, flips):
        self.bb = bb
        self.flips = frozenset(flips)
        self.root = dict(token=int(anchor), score=0.0, ranks=(), depth=0, parent=None)
        self.frontier = [self.root]
        self.candidates = []
        self.boundaries = []  # (boundary id, oracle gap)

    def step(self, d, D, Z, k, F):
        V = Z.shape[1]
        kk = min(k, V)
        children = []
        for m, u in enumerate(self.frontier):
            z = Z[m]
            lse = float(logsumexp(z))
            ids, vals = top_k(z, kk + 1 if kk < V else kk)
            pick = list(range(kk))
            if kk < V:
                bid = ("topk", u["ranks"])
                self.boundaries.append((bid, float(vals[kk - 1] - vals[kk])))
                if bid in self.flips:
                    pick[kk - 1] = kk
            for j, q in enumerate(pick):
                children.append(dict(token=int(ids[q]), score=u["score"] + (float(vals[q]) - lse),
                                     ranks=u["ranks"] + (j,), depth=d, parent=u))
        self.candidates.extend(children)
        if d < D:
            children.sort(key=_order_key)
            if len(children) > F:
                bid = ("frontier", d)
                self.boundaries.append((bid, children[F - 1]["score"] - children[F]["score"]))
                self.frontier = (children[:F - 1] + [children[F]] if bid in self.flips
                                 else children[:F])
            else:
                self.frontier = children

    def pack(self, N):
        cands = sorted(self.candidates, key=_order_key)
        if len(cands) > N:
            bid = ("pack",)
            self.boundaries.append((bid, cands[N - 1]["score"] - cands[N]["score"]))
            packed = cands[:N - 1] + [cands[N]] if bid in self.flips else cands[:N]
        else:
            packed = cands[:N]
        pos = {id(self.root): 0}
        for j, c in enumerate(packed):
            pos[id(c)] = j + 1
        tokens = np.full(N, -1, dtype=np.int32)
        parents = np.full(N, -1, dtype=np.int32)
        logq = np.full(N, -np.inf, dtype=np.float64)
        depths = np.zeros(N, dtype=np.int32)
        for j, c in enumerate(packed):
            tokens[j] = c["token"]
            parents[j] = pos[id(c["parent"])]
            logq[j] = c["score"]
            depths[j] = c["depth"]
        return dict(tree_tokens=tokens, parents=parents, logq=logq, depths=depths,
                    num_nodes=len(packed))


def _expand_jobs(jobs, W: np.ndarray, E, *, k: int, F: int, N: int):
    """Run the expansions of several requests depth by depth; one matmul per
    depth covers every job's frontier (the same float64 arithmetic per parent)."""
    D = jobs[0].bb.shape[0]
    for d in range(1, D + 1):
        rows = [E(u["token"]) for j in jobs for u in j.frontier]
        Z = parent_logits(np.zeros(W.shape[0]), W, np.stack(rows))
        at = 0
        for j in jobs:
            m = len(j.frontier)
            j.step(d, D, Z[at:at + m] + j.bb[d - 1][None, :], k, F)
            at += m
    return [j.pack(N) for j in jobs]


def expand_request(bb: np.ndarray, W: np.ndarray, E, anchor: int, *, k: int, F: int,
                   N: int, diag: dict | None = None, flips=()):
    """One request. bb [D, V] float64 backbone logits, W [V, H] float64, E(t) the
    float64 embedding row of token t; flips: boundary ids taken the other way.

    Returns (tree_tokens [N], parents [N], logq [N], depths [N], num_nodes);
    entries past num_nodes hold -1, -1, -inf, 0.
    """
    job = _Job(bb, anchor, flips)
    t = _expand_jobs([job], W, E, k=k, F=F, N=N)[0]
    if diag is not None:
        _fill_diag(diag, job)
    return t["tree_tokens"], t["parents"], t["logq"], t["depths"], t["num_nodes"]


def _fill_diag(diag, job):
    diag["candidates"] = len(job.candidates)
    diag["boundaries"] = list(job.boundaries)
    diag["topk_gaps"] = [g for b, g in job.boundaries if b[0] == "topk"]
    diag["frontier_gaps"] = [g for b, g in job.boundaries if b[0] == "frontier"]
    pg = [g for b, g in job.boundaries if b[0] == "pack"]
    diag["pack_gap"] = pg[0] if pg else np.inf
    diag["scores"] = [c["score"] for c in job.candidates]


def expand(backbone_bits: np.ndarray, W_bits: np.ndarray, E_bits: np.ndarray, anchor: np.ndarray, *,
           k: int = 4, F: int = 4, N: int = 32, requests=None, diags: list | None = None,
           W64: np.ndarray | None = None):
    """Batch of requests (bf16 bit inputs). requests: indices to compute (default all).

    Returns dict of arrays [len(requests), N] and num_nodes [len(requests)].
    W64: the head's float64 widening if the caller already holds it.
    """
    reqs = range(backbone_bits.shape[0]) if requests is None else list(requests)
    W = bf16_to_f64(W_bits) if W64 is None else W64
    E = lambda t: bf16_to_f64(E_bits[t])
    jobs = [_Job(bf16_to_f64(backbone_bits[b]), int(anchor[b]), ()) for b in reqs]
    trees = _expand_jobs(jobs, W, E, k=k, F=F, N=N)
    if diags is not None:
        for j in jobs:
            dg = {}
            _fill_diag(dg, j)
            diags.append(dg)
    return {key: np.asarray([t[key] for t in trees]) for key in trees[0]} if trees else {}


def near_tie_variants(backbone_bits: np.ndarray, W_bits: np.ndarray, E_bits: np.ndarray,
                      anchor: int, b: int, diag: dict, *, k: int, F: int, N: int,
                      excuse: float = 1e-5, max_flips: int = 2, W64: np.ndarray | None = None):
    """The request's trees with one or two near-tie boundaries (gap < excuse)
    taken the other way: a list of (label, tree dict)."""
    near = [bid for bid, g in diag["boundaries"] if g < excuse]
    sets = [(x,) for x in near]
    if max_flips >= 2:
        sets += [(x, y) for i, x in enumerate(near) for y in near[i + 1:]]
    if not sets:
        return []
    W = bf16_to_f64(W_bits) if W64 is None else W64
    E = lambda t: bf16_to_f64(E_bits[t])
    bb = bf16_to_f64(backbone_bits[b])
    jobs = [_Job(bb, anchor, s) for s in sets]
    trees = _expand_jobs(jobs, W, E, k=k, F=F, N=N)
    return [("+".join(x[0] for x in s), t) for s, t in zip(sets, trees)]
