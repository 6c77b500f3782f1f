"""Float64 CPU oracle of the fixed-branching beam tree on SparklingTree's
conditioned rows.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the product path.
Shares no code with the HIP library (it builds on the SparklingTree oracle's
conditioned rows, oracle/sparkling.py).

What it computes (SparklingTree post, "Future Ideas", item 4: a beam with a
fixed branching budget instead of the best-first heap, with the branches
spread evenly over the depths): the drafter rows and the Markov head give
the same conditioned rows as SparklingTree (top C candidates per row; a
child row is conditioned on its parent's token; log-probs over the C
candidates). Depth by depth, the beam keeps the w_d best children of the
previous depth's beam.

Readings of what the post leaves open (plainest consistent ones):
  * the branching budget is a per-depth width schedule w_1..w_L (the tree
    has sum w_d nodes); "evenly spread" is the default schedule, the budget
    B split as evenly as possible with the remainder on the first depths;
  * depth 1 takes the w_1 best children of the root row; depth d+1 takes
    the w_{d+1} best of all children of depth d's beam nodes;
  * "best" = score desc, then rank tuple lexicographic asc (the rank of a
    child is its position in its conditioned row, lp desc, token asc), as
    for SparklingTree; score = sum of lp along the path in float64;
  * a width above the number of candidates keeps them all; an empty depth
    ends the tree;
  * the tree is emitted depth by depth, each depth in beam order, so a
    parent precedes its children; node j+1 is the j-th emitted node.

Near-tie variants: each depth's cut (its w-th and (w+1)-th candidates) is
recorded with its gap; a variant keeps the (w+1)-th in place of the w-th at
the given depths and continues with the same arithmetic. The parity check
compares a device tree with the variants of cuts closer than 1e-5.
"""

from __future__ import annotations

import numpy as np

from oracle import sparkling as S


def even_widths(B: int, L: int) -> list[int]:
    """The budget B split over L depths as evenly as possible (remainder first)."""
    q, r = divmod(B, L)
    return [q + (1 if d < r else 0) for d in range(L)]


def build_request(x: np.ndarray, W1: np.ndarray, W2t: np.ndarray, widths, C: int, diag=None,
                  flips=(), rows=None):
    rows = S.Rows(x, W1, W2t, C) if rows is None else rows
    L = rows.L
    beam = [((), None, 0.0, 0)]  # (rank tuple, token, score, node number)
    tokens, parents, logq, depths = [], [], [], []
    cut_gaps = []
    for d in range(L):
        w = int(widths[d])
        cands = []
        for ranks, tok, sc, node in beam:
            ct, cl = rows.row(d, tok)
            for r in range(ct.shape[0]):
                cands.append((sc + float(cl[r]), ranks + (r,), int(ct[r]), node))
        cands.sort(key=lambda c: (-c[0], c[1]))
        if w < len(cands) and w > 0:
            cut_gaps.append((d, cands[w - 1][0] - cands[w][0]))
            kept = cands[:w - 1] + [cands[w]] if d in flips else cands[:w]
        else:
            kept = cands[:w]
        beam = []
        for sc, ranks, tok, par in kept:
            tokens.append(tok)
            parents.append(par)
            logq.append(sc)
            depths.append(d + 1)
            beam.append((ranks, tok, sc, len(tokens)))
        if not beam:
            break
    if diag is not None:
        diag["cut_gaps"] = [g for _, g in cut_gaps]
        diag["cuts"] = cut_gaps
        diag["rows"] = rows
    return tokens, parents, logq, depths


def build(logits_bits: np.ndarray, W1_bits: np.ndarray, W2t_bits: np.ndarray, widths, C: int,
          requests=None, diags: list | None = None) -> dict:
    """Batch of requests from bf16 bits: logits [batch, L, V], W1 / W2t [V, R];
    outputs padded to B = sum(widths) like the other trees."""
    reqs = range(logits_bits.shape[0]) if requests is None else list(requests)
    W1, W2t = S.bf16_to_f64(W1_bits), S.bf16_to_f64(W2t_bits)
    B = int(sum(widths))
    out = dict(tree_tokens=[], parents=[], logq=[], depths=[], num_nodes=[])
    for b in reqs:
        dg = {} if diags is not None else None
        t, p, q, dep = build_request(S.bf16_to_f64(logits_bits[b]), W1, W2t, widths, C, diag=dg)
        if diags is not None:
            diags.append(dg)
        n = len(t)
        pad = B - n
        out["tree_tokens"].append(np.array(t + [-1] * pad, np.int32))
        out["parents"].append(np.array(p + [-1] * pad, np.int32))
        out["logq"].append(np.array(q + [-np.inf] * pad, np.float64))
        out["depths"].append(np.array(dep + [0] * pad, np.int32))
        out["num_nodes"].append(n)
    return {k: np.asarray(v) for k, v in out.items()}


def near_tie_variants(x_bits: np.ndarray, W1_bits: np.ndarray, W2t_bits: np.ndarray, widths,
                      C: int, diag: dict, excuse: float = 1e-5, max_flips: int = 2):
    """The request's beam trees with one or two near-tie cuts (gap < excuse)
    taken the other way: a list of (label, tree dict). diag is the request's
    diagnostics from build (its conditioned rows are reused)."""
    near = [d for d, g in diag["cuts"] if g < excuse]
    sets = [(d,) for d in near]
    if max_flips >= 2:
        sets += [(a, c) for i, a in enumerate(near) for c in near[i + 1:]]
    B = int(sum(widths))
    out = []
    for s in sets:
        t, p, q, dep = build_request(None, None, None, widths, C, flips=s, rows=diag["rows"])
        n = len(t)
        pad = B - n
        out.append(("cut@" + ",".join(str(d + 1) for d in s),
                    dict(tree_tokens=np.array(t + [-1] * pad, np.int32),
                         parents=np.array(p + [-1] * pad, np.int32),
                         logq=np.array(q + [-np.inf] * pad, np.float64),
                         depths=np.array(dep + [0] * pad, np.int32), num_nodes=n)))
    return out
