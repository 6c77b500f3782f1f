"""Helpers shared by the GPU parity tests: device transfer and tree comparison.

Tree comparison follows the parity rule for this path: token and parent
indices must match exactly; log-probabilities within 1e-4. A mismatch is
excused only in two counted classes:
  E1  the node sets differ and the oracle's B-th and (B+1)-th prefix scores
      differ by less than 1e-5 (but not by exactly 0: an exact tie is decided
      by the rank-tuple rule, identically on both sides);
  E2  the node sets agree and only prefixes of different depths whose oracle
      scores differ by less than 1e-5 appear in a different order.
Everything else is a failure.
"""

from __future__ import annotations

import numpy as np
import torch

EXCUSE = 1e-5
LOGQ_TOL = 1e-4


def to_device(x: np.ndarray, dtype_code: int, device="cuda:0") -> torch.Tensor:
    if dtype_code == 0:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host(d: dict) -> dict:
    out = {}
    for k, v in d.items():
        a = v.cpu().numpy()
        out[k] = a.view(np.uint64) if k == "mask" else a
    return out


def paths(tok, par, n):
    P = {0: ()}
    for j in range(n):
        P[j + 1] = P[int(par[j])] + (int(tok[j]),)
    return [P[j + 1] for j in range(n)]


def classify(g: dict, o: dict, b: int, B: int) -> str:
    ng, no = int(g["num_nodes"][b]), int(o["num_nodes"][b])
    if ng != no:
        return f"F:count {ng} vs {no}"
    same = (np.array_equal(g["tree_tokens"][b], o["tree_tokens"][b])
            and np.array_equal(g["parents"][b], o["parents"][b])
            and ("depths" not in g or np.array_equal(g["depths"][b], o["depths"][b])))
    if same:
        d = np.abs(g["logq"][b, :no].astype(np.float64) - o["logq"][b, :no].astype(np.float64))
        if no and d.max() > LOGQ_TOL:
            return f"F:logq {d.max():.3g}"
        if not np.all(g["tree_tokens"][b, no:] == -1) or not np.all(g["parents"][b, no:] == -1):
            return "F:padding"
        return "exact"
    pg = paths(g["tree_tokens"][b], g["parents"][b], ng)
    po = paths(o["tree_tokens"][b], o["parents"][b], no)
    so = {p: float(s) for p, s in zip(po, o["score64"][b, :no])}
    lg = {p: float(v) for p, v in zip(pg, g["logq"][b, :ng])}
    for p in set(pg) & set(po):
        if abs(lg[p] - so[p]) > LOGQ_TOL:
            return f"F:logq {p}"
    if set(pg) != set(po):
        gap = float(o["score64"][b, B - 1] - o["next_score"][b]) if no == B else np.inf
        if 0.0 < gap < EXCUSE:
            return "E1"
        return f"F:set gap={gap:.3g} diff={len(set(pg) ^ set(po))}"
    pos = {p: i for i, p in enumerate(pg)}
    for i in range(no):
        for j in range(i + 1, no):
            a, c = po[i], po[j]  # oracle order a before c
            if pos[a] > pos[c]:
                if not (len(a) != len(c) and abs(so[a] - so[c]) < EXCUSE):
                    return f"F:order {a} {c}"
    return "E2"


def compare_batch(g: dict, o: dict, B: int, idx=None) -> dict:
    """Classify every request; idx maps oracle rows to GPU rows (default same)."""
    counts = {}
    fails = []
    n = len(o["num_nodes"])
    for i in range(n):
        gb = i if idx is None else idx[i]
        gi = {k: v[gb:gb + 1] for k, v in g.items()}
        oi = {k: v[i:i + 1] for k, v in o.items()}
        c = classify(gi, oi, 0, B)
        key = c if not c.startswith("F") else "F"
        counts[key] = counts.get(key, 0) + 1
        if c.startswith("F"):
            fails.append((gb, c))
    return dict(counts=counts, fails=fails)
