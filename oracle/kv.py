"""CPU oracle of KV-cache compaction to the accepted path.

TEST INFRASTRUCTURE ONLY: imported by tests/ and bench.py's cpu_baseline
leg, never by the product path. Shares no code with the HIP library.

What it computes (DDTree explainer, section 5, "KV cache management"): after
each round only the accepted path's cache is kept. Reading of the pages
(plainest consistent one): the verification pass wrote the key and value
rows of the tree's nodes at positions past + j (j = 0 the root, i.e. the
bonus token, j = 1..B the nodes in output order). After the walk accepted
the nodes a_1..a_n (node numbers, a path from the root), rows past + i for
i = 1..n take the rows of node a_i, the root's row stays, and the cache's
length becomes past + n + 1. Every other row is left as it was.

Layout: k, v [layers][batch][heads][cap][dh] (any element type, copied
bit for bit).
"""

from __future__ import annotations

import numpy as np


def compact(k: np.ndarray, v: np.ndarray, past_len: np.ndarray, accepted: np.ndarray,
            accept_len: np.ndarray):
    """Returns (k', v', new_len) without modifying the inputs.

    accepted [batch][L] node numbers (-1 padded), accept_len [batch].
    """
    k2, v2 = k.copy(), v.copy()
    batch = k.shape[1]
    new_len = np.empty(batch, dtype=np.int32)
    for b in range(batch):
        past, n = int(past_len[b]), int(accept_len[b])
        for i in range(1, n + 1):
            src = past + int(accepted[b, i - 1])
            # the source rows come from the cache as the verification left it
            k2[:, b, :, past + i, :] = k[:, b, :, src, :]
            v2[:, b, :, past + i, :] = v[:, b, :, src, :]
        new_len[b] = past + n + 1
    return k2, v2, new_len
