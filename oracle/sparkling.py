"""Float64 CPU oracle of SparklingTree's conditioned best-first tree.

TEST INFRASTRUCTURE ONLY: imported by tests/ and bench.py's cpu_baseline
leg, never by the product path. Shares no code with the HIP library.

What it computes (SparklingTree post, "Building SparklingTree" and "Solving
the candidate tree construction"): the diffusion drafter's rows x_d are cut
to their top C tokens on the device (a lossy pre-filter the post accepts);
a first-order Markov head biases row d+1 by the token chosen at depth d,
delta(p, v) = W1[p] . W2[:, v] (a rank-R factorisation: extraction W1
[V][R], projection W2 [R][V], here held transposed as W2t [V][R]); trees
grow best first: pop the best prefix, push its best child (the child row
conditioned on the popped token, re-sorted) and its next sibling (already
sorted and conditioned), until the budget is spent.

Readings of what the post leaves open (plainest consistent ones):
  * depth 1 is not conditioned (the outline sorts the first row directly and
    conditions depth i+1 on depth i);
  * a row's log-probs are taken over its C candidates: lp_j = s_j -
    logsumexp(s) with s_j = x_{d}[c_j] + delta(p, c_j) (delta = 0 at depth
    1), since the pre-filter hands on only those C entries;
  * inside a row children sort by (lp desc, token id asc); prefixes by
    (score desc, rank tuple lexicographic asc), a prefix before its
    extensions, score = sum of lp along the path (float64, left to right),
    as for DDTree.
Outputs follow DDTree's numbering: node j+1 is the j-th pop, parents[j] its
parent's node number (0 = root), logq its score, depths its depth.
"""

from __future__ import annotations

import heapq

import numpy as np
from scipy.special import logsumexp


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def top_c(row: np.ndarray, C: int) -> np.ndarray:
    """Token ids of the C largest entries by (value desc, id asc)."""
    return np.lexsort((np.arange(row.shape[0]), -row))[:C]


class Rows:
    """The conditioned child rows of one request (computed on first use)."""

    def __init__(self, x: np.ndarray, W1: np.ndarray, W2t: np.ndarray, C: int):
        self.x, self.W1, self.W2t = x, W1, W2t
        self.L = x.shape[0]
        self.cand = [top_c(x[d], min(C, x.shape[1])) for d in range(self.L)]
        self.cache = {}

    def row(self, d: int, parent_token):
        """Children at depth index d (0-based) of a node holding parent_token
        (None at depth 0): (tokens, lp) sorted by (lp desc, token asc)."""
        key = (d, parent_token)
        if key not in self.cache:
            c = self.cand[d]
            s = self.x[d, c].copy()
            if parent_token is not None:
                s = s + self.W2t[c] @ self.W1[parent_token]
            lp = s - logsumexp(s)
            order = np.lexsort((c, -lp))
            self.cache[key] = (c[order], lp[order])
        return self.cache[key]


def build_request(x: np.ndarray, W1: np.ndarray, W2t: np.ndarray, B: int, C: int, diag=None):
    """One request: x [L, V] float64 logits, W1 / W2t [V, R] float64."""
    R = Rows(x, W1, W2t, C)
    toks, lps = R.row(0, None)
    # heap entries: (-score, rank tuple, node id); nodes: (depth, rank, token, score, parent node)
    nodes = []
    heap = []

    def push(depth, ranks, token, score, parent, row):
        nodes.append(dict(depth=depth, ranks=ranks, token=token, score=score, parent=parent, row=row))
        heapq.heappush(heap, (-score, ranks, len(nodes) - 1))

    push(1, (0,), int(toks[0]), float(lps[0]), -1, (toks, lps))
    out_pos = {}
    tokens, parents, logq, depths = [], [], [], []
    pops = []
    while heap and len(tokens) < B:
        negs, ranks, nid = heapq.heappop(heap)
        nd = nodes[nid]
        out_pos[nid] = len(tokens) + 1
        tokens.append(nd["token"])
        parents.append(0 if nd["parent"] < 0 else out_pos[nd["parent"]])
        logq.append(nd["score"])
        depths.append(nd["depth"])
        pops.append(-negs)
        # sibling: the next entry of the same (conditioned, sorted) row
        st, sl = nd["row"]
        r = ranks[-1] + 1
        if r < st.shape[0]:
            base = 0.0 if nd["parent"] < 0 else nodes[nd["parent"]]["score"]
            push(nd["depth"], ranks[:-1] + (r,), int(st[r]), base + float(sl[r]), nd["parent"],
                 nd["row"])
        # child: the best entry of the row conditioned on this node's token
        if nd["depth"] < R.L:
            ct, cl = R.row(nd["depth"], nd["token"])
            push(nd["depth"] + 1, ranks + (0,), int(ct[0]), nd["score"] + float(cl[0]), nid, (ct, cl))
    n = len(tokens)
    pad = B - n
    if diag is not None:
        diag["pops"] = pops
        diag["next_score"] = -heap[0][0] if heap else -np.inf
        diag["rows"] = R
    return (np.array(tokens + [-1] * pad, np.int32), np.array(parents + [-1] * pad, np.int32),
            np.array(logq + [-np.inf] * pad, np.float64), np.array(depths + [0] * pad, np.int32), n)


def build(logits_bits: np.ndarray, W1_bits: np.ndarray, W2t_bits: np.ndarray, B: int, C: int,
          requests=None, diags: list | None = None) -> dict:
    """Batch of requests from bf16 bits: logits [batch, L, V], W1 / W2t [V, R]."""
    reqs = range(logits_bits.shape[0]) if requests is None else list(requests)
    W1, W2t = bf16_to_f64(W1_bits), bf16_to_f64(W2t_bits)
    out = dict(tree_tokens=[], parents=[], logq=[], depths=[], num_nodes=[])
    for b in reqs:
        dg = {} if diags is not None else None
        t, p, q, dep, n = build_request(bf16_to_f64(logits_bits[b]), W1, W2t, B, C, diag=dg)
        if diags is not None:
            diags.append(dg)
        for k, v in zip(("tree_tokens", "parents", "logq", "depths", "num_nodes"), (t, p, q, dep, n)):
            out[k].append(v)
    return {k: np.asarray(v) for k, v in out.items()}
