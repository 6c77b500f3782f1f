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


def expand_request(bb: np.ndarray, W: np.ndarray, E, anchor: int, *, k: int, F: int,
                   N: int, diag: dict | None = None):
    """One request. bb [D, V] float64 backbone logits, W [V, H] float64, E(t) the
    float64 embedding row of token t.

    Returns (tree_tokens [N], parents [N], logq [N], depths [N], num_nodes);
    entries past num_nodes hold -1, -1, -inf, 0.
    """
    D, V = bb.shape
    kk = min(k, V)
    root = dict(token=int(anchor), score=0.0, ranks=(), depth=0, parent=None)
    frontier = [root]
    candidates = []
    gaps = []  # per-parent k-th minus (k+1)-th z (excuse boundaries)
    fgaps = []  # per depth: F-th minus (F+1)-th child score (frontier boundary)
    for d in range(1, D + 1):
        E_rows = np.stack([E(u["token"]) for u in frontier])
        Z = parent_logits(bb[d - 1], W, E_rows)
        children = []
        for m, u in enumerate(frontier):
            z = Z[m]
            lse = float(logsumexp(z))
            ids, vals = top_k(z, kk + 1 if kk < V else kk)
            if kk < V:
                gaps.append(float(vals[kk - 1] - vals[kk]))
            for j in range(kk):
                children.append(dict(token=int(ids[j]), score=u["score"] + (float(vals[j]) - lse),
                                     ranks=u["ranks"] + (j,), depth=d, parent=u))
        candidates.extend(children)
        if d < D:
            children.sort(key=_order_key)
            if len(children) > F:
                fgaps.append(children[F - 1]["score"] - children[F]["score"])
            frontier = children[:F]
    candidates.sort(key=_order_key)
    packed = candidates[:N]
    pos = {id(root): 0}
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
    if diag is not None:
        diag["candidates"] = len(candidates)
        diag["topk_gaps"] = gaps
        diag["frontier_gaps"] = fgaps
        diag["pack_gap"] = (candidates[N - 1]["score"] - candidates[N]["score"]
                            if len(candidates) > N else np.inf)
        diag["scores"] = [c["score"] for c in candidates]
    return tokens, parents, logq, depths, len(packed)


def expand(backbone_bits: np.ndarray, W_bits: np.ndarray, E_bits: np.ndarray, anchor: np.ndarray, *,
           k: int = 4, F: int = 4, N: int = 32, requests=None, diags: list | None = None):
    """Batch of requests (bf16 bit inputs). requests: indices to compute (default all).

    Returns dict of arrays [len(requests), N] and num_nodes [len(requests)].
    """
    reqs = range(backbone_bits.shape[0]) if requests is None else list(requests)
    W = bf16_to_f64(W_bits)
    E = lambda t: bf16_to_f64(E_bits[t])
    out = dict(tree_tokens=[], parents=[], logq=[], depths=[], num_nodes=[])
    for b in reqs:
        dg = {} if diags is not None else None
        t, p, q, dep, n = expand_request(bf16_to_f64(backbone_bits[b]), W, E, int(anchor[b]),
                                         k=k, F=F, N=N, diag=dg)
        if diags is not None:
            diags.append(dg)
        out["tree_tokens"].append(t)
        out["parents"].append(p)
        out["logq"].append(q)
        out["depths"].append(dep)
        out["num_nodes"].append(n)
    return {key: np.asarray(v) for key, v in out.items()}
