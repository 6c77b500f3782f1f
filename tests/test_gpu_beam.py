"""GPU parity of sparkling_beam against the float64 oracle (SparklingTree
post, "Future Ideas", item 4).

Device log-probs are float32 (as sparkling_build), the oracle's float64, so
trees must match exactly except in two counted classes:
  E1  the device tree is the oracle's tree with one or two depth cuts whose
      w-th and (w+1)-th candidates are closer than 1e-5 taken the other way
      (oracle/beam.py near_tie_variants), expanded on from there;
  E2  the same prefixes, and only prefixes whose oracle scores are < 1e-5
      apart appear in a different order.
logq within 1e-4 of the matching oracle tree; flat rows with a zero head
(exact ties everywhere, including the tie-extraction path) bit-exact."""

import numpy as np
import pytest
import torch

import draft_tree_construction_depth_amd as pkg
from draft_tree_construction_depth_amd import gen
from oracle import beam as BM
from oracle import oracle as O
from parity_util import classify_variants, record

pytestmark = pytest.mark.gpu

LOGQ_TOL = 1e-4


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(x, W1, W2t, widths, C):
    out = pkg.sparkling_beam(_dev_bf16(x), _dev_bf16(W1), _dev_bf16(W2t), widths, C=C)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    g["mask"] = g["mask"].view(np.uint64)
    return g


def _compare(g, o, diags, rows, B, label, x, W1, W2t, widths, C):
    counts = {}
    for i, gb in enumerate(rows):
        gi = {k: g[k][gb] for k in ("tree_tokens", "parents", "logq", "depths", "num_nodes")}
        ref = {k: o[k][i] for k in ("tree_tokens", "parents", "logq", "depths", "num_nodes")}
        c = classify_variants(gi, [(None, ref)])
        if c.startswith("F"):
            c = classify_variants(gi, BM.near_tie_variants(x, W1, W2t, widths, C, diags[i]))
        assert not c.startswith("F"), f"request {gb}: {c}"
        key = c.split(":")[0]
        counts[key] = counts.get(key, 0) + 1
    record(label, counts)
    return counts


CASES = [
    # seed, batch, L, V, C, R, widths, wscale
    (0, 4, 5, 4096, 32, 64, [4, 4, 4, 4, 4], 0.3),
    (1, 3, 8, 3000, 64, 128, [8, 8, 8, 8, 8, 8, 8, 8], 0.2),
    (2, 3, 6, 3001, 40, 64, [1, 2, 4, 8, 16, 32], 0.3),    # back-loaded, unaligned rows
    (3, 2, 6, 2000, 16, 64, [32, 16, 8, 4, 2, 1], 0.3),    # front-loaded; depth 1 keeps all 16
    (4, 2, 15, 5000, 128, 256, BM.even_widths(64, 15), 0.177),
    (5, 2, 4, 500, 50, 64, [64, 64, 64, 64], 0.3),         # widest beams
    (6, 2, 5, 800, 8, 64, [3, 0, 5, 5, 5], 0.3),           # a zero width ends the tree
    (7, 70, 3, 700, 8, 64, [2, 3, 4], 0.5),                # many requests
    (8, 2, 1, 900, 16, 64, [7], 0.3),                      # one row
]


@pytest.mark.parametrize("seed,batch,L,V,C,R,widths,ws", CASES)
def test_beam_small(seed, batch, L, V, C, R, widths, ws):
    x, W1, W2t = gen.sparkling_inputs(seed, batch=batch, L=L, V=V, R=R, wscale=ws)
    diags = []
    o = BM.build(x, W1, W2t, widths, C, diags=diags)
    g = _run(x, W1, W2t, widths, C)
    B = sum(widths)
    st = _compare(g, o, diags, list(range(batch)), B, f"beam L={L} C={C} widths={widths}",
                  x, W1, W2t, widths, C)
    print(f"beam seed={seed} batch={batch} L={L} C={C} widths={widths}: {st}")
    np.testing.assert_array_equal(g["mask"], O.mask(g["parents"], g["num_nodes"], B))


@pytest.mark.parametrize("C,widths", [(64, [5, 40, 64]), (128, [1, 64, 64]), (8, [8, 64, 64, 64])])
def test_beam_flat_rows_exact(C, widths):
    """Flat rows, zero head: every candidate of a depth ties; the beam is the
    first rank tuples (64 x 128 tied candidates take the extraction path)."""
    L, V, R, batch = len(widths), 512, 64, 2
    x = np.zeros((batch, L, V), dtype=np.uint16)
    W = np.zeros((V, R), dtype=np.uint16)
    o = BM.build(x, W, W, widths, C)
    g = _run(x, W, W, widths, C)
    for b in range(batch):
        n = int(o["num_nodes"][b])
        for k in ("tree_tokens", "parents", "depths", "num_nodes"):
            np.testing.assert_array_equal(g[k][b], o[k][b], err_msg=k)
        np.testing.assert_allclose(g["logq"][b][:n], o["logq"][b][:n], rtol=0, atol=LOGQ_TOL)


def test_beam_post_shape_sampled():
    """The batch-64 workload (15 rows of V = 151936, C = 128, R = 256) with
    B = 64 spread evenly, in one launch; eight requests against the oracle."""
    c = gen.SPARKLING
    x, W1, W2t = gen.sparkling_inputs(0)
    widths = BM.even_widths(c["B"], c["L"])
    g = _run(x, W1, W2t, widths, c["C"])
    rows = list(range(0, 64, 8))
    diags = []
    o = BM.build(x, W1, W2t, widths, c["C"], requests=rows, diags=diags)
    xs = x[rows]
    st = _compare(g, o, diags, rows, c["B"], "beam batch-64 workload (8 of 64 requests)",
                  xs, W1, W2t, widths, c["C"])
    print(f"beam batch-64 workload, requests {rows}: {st}")
    assert (g["num_nodes"] == c["B"]).all()
    for b in range(c["batch"]):
        dep = g["depths"][b]
        assert [int((dep == d + 1).sum()) for d in range(c["L"])] == widths


def test_beam_default_schedule_is_the_even_split():
    """widths None: the library spreads the budget itself; the same trees as
    the explicit even schedule."""
    x, W1, W2t = gen.sparkling_inputs(12, batch=3, L=7, V=3000, R=64, wscale=0.3)
    a = pkg.sparkling_beam(_dev_bf16(x), _dev_bf16(W1), _dev_bf16(W2t), B=30, C=32)
    b = pkg.sparkling_beam(_dev_bf16(x), _dev_bf16(W1), _dev_bf16(W2t), BM.even_widths(30, 7),
                           C=32)
    torch.cuda.synchronize()
    for k in a:
        np.testing.assert_array_equal(a[k].cpu().numpy(), b[k].cpu().numpy(), err_msg=k)
    dep = a["depths"].cpu().numpy()
    assert [int((dep[0] == d + 1).sum()) for d in range(7)] == BM.even_widths(30, 7)
