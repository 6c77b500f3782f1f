"""GPU parity of treespark_expand against the float64 oracle (TreeSpark
README, items 1-2). A tree must equal the oracle's (order swaps of nodes
< 1e-5 apart counted as E2) or one of the oracle's trees with one or two
boundaries -- a parent's k-th/(k+1)-th child, a frontier cut, the packing
cut -- closer than 1e-5 taken the other way (E1, z is accumulated in float32
on the device); logq within 1e-4 of the matching tree."""

import numpy as np
import pytest
import torch

import draft_tree_construction_depth_amd as pkg
from draft_tree_construction_depth_amd import gen
from oracle import oracle as O
from oracle import treespark as T
from parity_util import classify_variants, record

pytestmark = pytest.mark.gpu

def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run_gpu(bb, W, E, anc, k, F, N, repeats=0):
    """One expansion; with repeats, that many more calls on the same device
    inputs and output buffers, each compared bit for bit with the first."""
    args = (_dev_bf16(bb), _dev_bf16(W), _dev_bf16(E), torch.from_numpy(anc.astype(np.int32)).cuda())
    out = pkg.treespark_expand(*args, k=k, F=F, N=N)
    first = {key: v.clone() for key, v in out.items()}
    for i in range(repeats):
        pkg.treespark_expand(*args, k=k, F=F, N=N, out=out)
        for key in first:
            assert torch.equal(first[key], out[key]), f"repeat {i}: {key} differs"
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in first.items()}


def _classify(o, g, diags, rows, label, bb, W, E, anc, k, F, N, W64=None):
    """rows: GPU batch indices matching the oracle's entries in order. A tree
    that differs from the oracle's must equal one of its near-tie variants."""
    stats = {}
    for i, b in enumerate(rows):
        gi = {key: g[key][b] for key in ("tree_tokens", "parents", "logq", "depths", "num_nodes")}
        ref = {key: o[key][i] for key in ("tree_tokens", "parents", "logq", "depths", "num_nodes")}
        c = classify_variants(gi, [(None, ref)])
        if c.startswith("F"):
            c = classify_variants(gi, T.near_tie_variants(bb, W, E, int(anc[b]), b, diags[i], k=k,
                                                          F=F, N=N, W64=W64))
        assert not c.startswith("F"), f"request {b}: {c}"
        stats[c] = stats.get(c, 0) + 1
    record(label, {key.split(":")[0]: v for key, v in stats.items()})
    return stats


CASES = [
    # seed, batch, D, V, H, k, F, N, wscale
    (0, 2, 4, 300, 64, 4, 4, 32, 0.3),
    (1, 3, 7, 1000, 128, 4, 4, 32, 0.1),
    (2, 4, 3, 777, 64, 2, 3, 10, 0.3),    # ragged vocabulary tile
    (3, 2, 1, 129, 64, 4, 4, 32, 0.3),    # one depth
    (4, 2, 5, 3, 64, 4, 4, 40, 0.3),      # V < k
    (5, 40, 3, 500, 64, 4, 4, 32, 0.3),   # 160 parents: two column blocks
    (6, 2, 16, 200, 64, 2, 2, 64, 0.3),   # deepest supported tree
    (7, 2, 4, 400, 192, 8, 8, 100, 0.3),  # k = F = 8
]


@pytest.mark.parametrize("seed,batch,D,V,H,k,F,N,ws", CASES)
def test_treespark_small(seed, batch, D, V, H, k, F, N, ws):
    bb, W, E, anc = gen.treespark_inputs(seed, batch=batch, D=D, V=V, H=H, wscale=ws)
    diags = []
    o = T.expand(bb, W, E, anc, k=k, F=F, N=N, diags=diags)
    g = _run_gpu(bb, W, E, anc, k, F, N)
    st = _classify(o, g, diags, list(range(batch)), f"treespark D={D} V={V} H={H} k={k} F={F} N={N}",
                   bb, W, E, anc, k, F, N)
    print(f"treespark seed={seed} batch={batch} D={D} V={V} H={H} k={k} F={F} N={N}: {st}")


def test_treespark_readme_shape_sampled():
    """The README's shape: 32 requests, 7 depths, V = 151936, H = 2560, k = 4,
    F = 4, N = 32; the oracle checks eight requests of the full launch, and
    20 more launches on the same inputs must repeat it bit for bit."""
    c = gen.TREESPARK
    bb, W, E, anc = gen.treespark_inputs(0)
    g = _run_gpu(bb, W, E, anc, c["k"], c["F"], c["N"], repeats=20)
    rows = list(range(0, 32, 4))
    diags = []
    W64 = T.bf16_to_f64(W)
    o = T.expand(bb, W, E, anc, k=c["k"], F=c["F"], N=c["N"], requests=rows, diags=diags, W64=W64)
    for dg in diags:
        assert dg["candidates"] == 100
    assert (g["num_nodes"] == 32).all()
    st = _classify(o, g, diags, rows, "treespark README shape (8 of 32 requests)", bb, W, E, anc,
                   c["k"], c["F"], c["N"], W64=W64)
    print(f"treespark README shape, requests {rows}: {st}")
    # structure of every request of the launch
    for b in range(c["batch"]):
        par, dep, lq = g["parents"][b], g["depths"][b], g["logq"][b]
        for j in range(32):
            assert 0 <= par[j] <= j
            assert dep[j] == (1 if par[j] == 0 else dep[par[j] - 1] + 1)
            assert lq[j] <= (0.0 if par[j] == 0 else lq[par[j] - 1]) + 1e-6


def test_treespark_mask():
    bb, W, E, anc = gen.treespark_inputs(3, batch=3, D=5, V=256, H=64, wscale=0.3)
    g = _run_gpu(bb, W, E, anc, 4, 4, 32)
    par = torch.from_numpy(g["parents"]).cuda()
    nn = torch.from_numpy(g["num_nodes"]).cuda()
    m = pkg.ddtree_mask(par, nn, 32)
    torch.cuda.synchronize()
    ref = O.mask(g["parents"], g["num_nodes"], 32)
    np.testing.assert_array_equal(m.cpu().numpy().view(np.uint64), ref)


@pytest.mark.parametrize("H,k,F,D", [(100, 4, 4, 3), (64, 9, 4, 3), (64, 4, 9, 3), (64, 4, 4, 17)])
def test_treespark_unsupported(H, k, F, D):
    bb, W, E, anc = gen.treespark_inputs(0, batch=1, D=min(D, 4), V=64, H=H)
    if D > 4:
        bb = np.concatenate([bb] * 5, axis=1)[:, :D]
    with pytest.raises(pkg.DDTreeError):
        _run_gpu(bb, W, E, anc, k, F, 8)
