"""Helpers shared by the GPU parity tests: device transfer, tree comparison
by excuse class (oracle/parity.py holds the rule) and the record of the
counts.

Counts of every compared configuration are kept for the session; when the
environment names a file in DDT_PARITY_JSON, conftest.py writes them there as
JSON at the end of the run.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle.parity import (EXCUSE, LOGQ_TOL, DDTreeScorer, RowsScorer,  # noqa: F401
                           classify_tree, classify_variants, ddtree_batch_counts)

RECORD: dict = {}


def record(label: str, counts: dict) -> None:
    """Add a configuration's class counts to the session record."""
    tot = RECORD.setdefault(label, {})
    for k, v in counts.items():
        tot[k] = tot.get(k, 0) + v


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


def classify(g: dict, o: dict, b: int, B: int) -> str:
    """Request b of a device batch g against request b of an oracle batch o."""
    r = ddtree_batch_counts({k: v[b:b + 1] for k, v in g.items()},
                            {k: v[b:b + 1] for k, v in o.items()}, B)
    return "F" if r["fails"] else next(iter(r["counts"]))


def compare_batch(g: dict, o: dict, B: int, idx=None) -> dict:
    """Classify every request; idx maps oracle rows to GPU rows (default same)."""
    return ddtree_batch_counts(g, o, B, idx)
