"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every input is seeded and synthetic (draft_tree_construction_depth_amd.gen).
Trees must match exactly up to the counted excuse classes of parity_util;
stage-1 ids and values are bit-exact, row normalisers within 2e-6; masks and
walks are bit-exact. The largest cases run at the full sizes of the workloads
(batch 64 / 256, V = 151936) in the same launch configuration as bench.py.
"""

from __future__ import annotations

import functools
import math
import os

import numpy as np
import pytest
import torch

import draft_tree_construction_depth_amd as pkg
from draft_tree_construction_depth_amd import gen
from oracle import oracle as O
from parity_util import classify, compare_batch, record, to_device, to_host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32, BF16 = gen.DTYPE_F32, gen.DTYPE_BF16
THREADS = max(1, min(16, os.cpu_count() or 1))


def _say(*a):
    print(*a, flush=True)


@functools.lru_cache(maxsize=8)
def _inputs(cfg, seed, batch=None, first=0):
    return gen.make_logits(cfg, seed, batch=batch, first=first)


@functools.lru_cache(maxsize=8)
def _oracle(cfg, seed, batch=None, first=0):
    c = gen.CONFIGS[cfg]
    return O.build(_inputs(cfg, seed, batch, first), c["dtype"], c["B"], threads=THREADS)


def _gpu_build(x, dt, B, **kw):
    out = pkg.ddtree_build(to_device(x, dt), B, **kw)
    torch.cuda.synchronize()
    return to_host(out)


# ----------------------------------------------------------------------------
# stage 1
# ----------------------------------------------------------------------------

ROW_CASES = [
    # rows, V, K, dtype, kind
    (3, 1024, 32, F32, "gauss"),
    (5, 1000, 64, BF16, "gauss"),
    (4, 5003, 128, BF16, "gauss"),      # row length not a multiple of 16 bytes
    (7, 40001, 256, F32, "gauss"),
    (2, 151936, 512, BF16, "gauss"),
    (3, 20000, 100, BF16, "ints"),      # heavy ties
    (2, 9000, 300, F32, "const"),       # every value tied
    (6, 3000, 1, BF16, "gauss"),
    (1, 7, 7, F32, "ints"),             # K == V
    (40, 151936, 128, BF16, "gauss"),
    (5, 30000, 64, BF16, "spike"),
    (3, 151936, 128, BF16, "straddle"),
    # >= 512 rows of 16-byte multiples: one workgroup per row
    (512, 8192, 128, BF16, "gauss"),
    (520, 6000, 64, BF16, "straddle"),
    (512, 4096, 256, BF16, "neg"),
    (600, 20000, 100, BF16, "ints"),
    (512, 2048, 128, BF16, "const"),   # more tied vectors than fit: exact path
    (512, 4096, 128, F32, "gauss"),
    (512, 151936, 256, BF16, "straddle"),
    (512, 151936, 256, BF16, "trend"),
    (512, 40000, 128, BF16, "zeros"),
]


def _rows(rows, V, dt, kind, seed=0):
    rng = np.random.default_rng(seed)
    if kind == "gauss":
        x = (rng.uniform(0.5, 8, (rows, 1)) * rng.standard_normal((rows, V))).astype(np.float32)
    elif kind in ("straddle", "neg"):
        # the top K values cross zero (straddle) or are all negative (neg)
        sig = rng.uniform(0.5, 8, (rows, 1))
        shift = 3.1 if kind == "straddle" else 40.0
        x = (sig * (rng.standard_normal((rows, V)) - shift)).astype(np.float32)
    elif kind == "trend":
        # rising along the row: early kept vectors go stale and get compacted
        sig = rng.uniform(0.5, 8, (rows, 1))
        x = (sig * (rng.standard_normal((rows, V)) + 8.0 * np.arange(V) / V)).astype(np.float32)
    elif kind == "ints":
        x = rng.integers(-3, 4, (rows, V)).astype(np.float32)
        x[:, :5] = -0.0
    elif kind == "zeros":
        # mostly -1 with about 1% each of -0 and +0 and 40 ones per row, so
        # the K-th value is zero: the threshold is exactly +0 while zeros
        # (many of them -0 beside nonzero neighbours) are still being kept
        u = rng.random((rows, V))
        x = np.where(u < 0.01, -0.0, np.where(u < 0.02, 0.0, -1.0)).astype(np.float32)
        for i in range(rows):
            x[i, rng.choice(V, 40, replace=False)] = 1.0
    elif kind == "spike":
        # one value 3e4 per row: the candidates' value codes span far more
        # than the merge's histogram holds (its bisection path)
        x = rng.standard_normal((rows, V)).astype(np.float32)
        x[np.arange(rows), rng.integers(0, V, rows)] = 3e4
    else:
        x = np.full((rows, V), 1.25, np.float32)
    return gen.f32_to_bf16_bits(x) if dt == BF16 else x


@pytest.mark.parametrize("case", ROW_CASES, ids=[f"{c[0]}x{c[1]}k{c[2]}d{c[3]}{c[4]}" for c in ROW_CASES])
def test_row_topk_matches_oracle(case):
    rows, V, K, dt, kind = case
    _say("row_topk", case)
    x = _rows(rows, V, dt, kind)
    r = pkg.ddtree_row_topk(to_device(x, dt), K)
    torch.cuda.synchronize()
    ids, vals, lse = (r[k].cpu().numpy() for k in ("ids", "vals", "lse"))
    for i in range(rows):
        oi, ov = O.row_rank(x[i], dt, K)
        np.testing.assert_array_equal(ids[i], oi, err_msg=f"row {i}")
        np.testing.assert_array_equal(vals[i].astype(np.float64), ov, err_msg=f"row {i}")
        assert abs(lse[i] - O.row_lse(x[i], dt)) < 2e-6


def test_row_topk_full_batch64_tables():
    # The 960 rows of the batch-64 workload, in its own launch configuration.
    x = _inputs(3, 0)
    o = _oracle(3, 0)
    _say("row_topk c3 full")
    r = pkg.ddtree_row_topk(to_device(x, BF16), 128)
    torch.cuda.synchronize()
    ids = r["ids"].cpu().numpy().reshape(64, 15, 128)
    vals = r["vals"].cpu().numpy().reshape(64, 15, 128)
    lse = r["lse"].cpu().numpy().reshape(64, 15)
    np.testing.assert_array_equal(ids, o["top_ids"])
    np.testing.assert_array_equal(vals.astype(np.float64), o["top_vals"])
    assert np.abs(lse - o["z"]).max() < 2e-6


# ----------------------------------------------------------------------------
# stage 2 (+3): whole build against the oracle; stage 4 on the device's trees
# ----------------------------------------------------------------------------

def _check_counts(res, label):
    record(label, res["counts"])
    _say(label, res["counts"])
    assert not res["fails"], f"{label}: {res['fails'][:5]}"


def _check_mask_of_own_parents(g, B):
    # the mask is a function of the parents: every request, excused or not
    np.testing.assert_array_equal(g["mask"], O.mask(g["parents"], g["num_nodes"], B))


def _walk_gpu_tree(g, tgt, L):
    """ddtree_accept on the device's own trees against the oracle's walk of
    the same trees and targets (bit-exact)."""
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    r = pkg.ddtree_accept(dv(g["tree_tokens"]), dv(g["parents"]), dv(g["num_nodes"]), dv(tgt), L)
    torch.cuda.synchronize()
    ga = [r[k].cpu().numpy() for k in ("accepted_nodes", "accept_len", "next_token")]
    oa = O.accept(g["tree_tokens"], g["parents"], g["num_nodes"], tgt, L)
    for a, b in zip(ga, oa):
        np.testing.assert_array_equal(a, b)
    return ga


def _drafter_targets(cfg, seed, x, g, B, first=0):
    Y = gen.drafter_draws(cfg, seed, x, gen.CONFIGS[cfg]["dtype"], first=first)
    return gen.node_targets_from_depths(Y, g["depths"], g["num_nodes"], B)


@pytest.mark.parametrize("seed", range(5))
def test_build_c1(seed):
    x = _inputs(1, seed)
    g = _gpu_build(x, F32, 32)
    o = _oracle(1, seed)
    res = compare_batch(g, o, 32)
    _check_counts(res, "batch-1 V=1024 f32 B=32")
    assert res["counts"].get("exact", 0) == 1
    np.testing.assert_array_equal(g["mask"], O.mask(o["parents"], o["num_nodes"], 32))


@pytest.mark.parametrize("seed", range(5))
def test_build_and_walk_c2(seed):
    x = _inputs(2, seed)
    g = _gpu_build(x, BF16, 64)
    o = _oracle(2, seed)
    _check_counts(compare_batch(g, o, 64), "batch-1 V=151936 bf16 B=64")
    _check_mask_of_own_parents(g, 64)
    _, alen, _ = _walk_gpu_tree(g, _drafter_targets(2, seed, x, g, 64), 15)
    _say("c2 seed", seed, "accept_len", int(alen[0]))


@pytest.mark.parametrize("seed", range(3))
def test_build_and_walk_c3_full_batch(seed):
    x = _inputs(3, seed)
    g = _gpu_build(x, BF16, 128)
    o = _oracle(3, seed)
    _check_counts(compare_batch(g, o, 128), "batch-64 V=151936 bf16 B=128")
    _check_mask_of_own_parents(g, 128)
    _, alen, _ = _walk_gpu_tree(g, _drafter_targets(3, seed, x, g, 128), 15)
    _say("c3 seed", seed, "mean accept_len", float(alen.mean()))


@pytest.mark.parametrize("seed", range(2))
def test_build_and_walk_c5_full_batch(seed):
    # All 256 trees of the batch-256 workload in its own launch shape; the
    # walk (B = 256: four register slots per lane) on every tree.
    x = gen.make_logits(5, seed)
    _say("c5 seed", seed, "inputs ready")
    g = _gpu_build(x, BF16, 256)
    o = O.build(x, BF16, 256, threads=THREADS)
    _check_counts(compare_batch(g, o, 256), "batch-256 V=151936 bf16 B=256")
    _check_mask_of_own_parents(g, 256)
    _, alen, _ = _walk_gpu_tree(g, _drafter_targets(5, seed, x, g, 256), 15)
    _say("c5 seed", seed, "mean accept_len", float(alen.mean()))


def test_build_c5_enumeration_overflow():
    # Request 15 of the batch-256 workload, seed 1, has 2436 prefixes at or
    # above its one-deviation threshold, more than the enumeration holds: the
    # threshold is raised to the B-th best entry found and the enumeration
    # restarts. Its neighbours take the ordinary path in the same launch.
    x = _inputs(5, 1, batch=3, first=14)
    g = _gpu_build(x, BF16, 256)
    o = O.build(x, BF16, 256, threads=THREADS)
    _check_counts(compare_batch(g, o, 256), "batch-256 requests 14-16 (enumeration overflow)")
    _check_mask_of_own_parents(g, 256)


@pytest.mark.parametrize("seed", range(1, 4))
def test_build_c3_small_batches(seed):
    # A few requests of the batch-64 workload (smaller launch shape).
    x = _inputs(3, seed, batch=3)
    g = _gpu_build(x, BF16, 128)
    o = _oracle(3, seed, batch=3)
    _check_counts(compare_batch(g, o, 128), "batch-64 workload, 3-request launches")


EDGE = [
    # name, L, V, B, dtype, kind
    ("V_below_B", 4, 20, 64, F32, "gauss"),
    ("budget_beyond_prefixes", 3, 3, 100, F32, "gauss"),
    ("L1", 1, 5000, 32, BF16, "gauss"),
    ("B1", 15, 5000, 1, BF16, "gauss"),
    ("const_rows", 6, 4000, 48, BF16, "const"),
    ("const_rows_V_below_B", 5, 30, 128, F32, "const"),
    ("int_ties", 8, 3001, 96, F32, "ints"),
    ("one_hot", 5, 1000, 40, F32, "onehot"),
    ("unaligned_V", 15, 10001, 128, BF16, "gauss"),
    ("L32_K8", 32, 8, 8, F32, "gauss"),
    ("B512_L13", 13, 5000, 512, BF16, "gauss"),
    # rank-tuple keys of 120 bits (L * ceil(log2 K) close to the 122-bit
    # bound) on full-depth trees whose deviations reach depth 8 and 16
    ("L30_K16_key120_chain", 30, 16, 48, F32, "chain"),
    ("L20_K64_key120_chain", 20, 3000, 64, BF16, "chain"),
    # the same chains against a -900 background: every other term of an odd
    # row underflows in the oracle's float64 normaliser, the dominant token's
    # log-probability is exactly 0 there and a prefix ties exactly with its
    # extension (a cross-depth tie the float32 normaliser need not reproduce)
    ("L30_K16_key120_chain_minus900", 30, 16, 48, F32, "chain900"),
    ("L20_K64_key120_chain_minus900", 20, 3000, 64, BF16, "chain900"),
]


def _edge_logits(L, V, dt, kind, batch, seed):
    rng = np.random.default_rng(seed)
    if kind == "gauss":
        x = (rng.uniform(0.3, 4, (batch, L, 1)) * rng.standard_normal((batch, L, V))).astype(np.float32)
    elif kind == "const":
        x = np.full((batch, L, V), -2.0, np.float32)
    elif kind == "ints":
        x = rng.integers(-2, 3, (batch, L, V)).astype(np.float32)
    else:
        # one dominant token per row; the chains make the runner-up on even
        # rows so unlikely that the tree's spine runs to depth L; "chain"
        # keeps the background at -30, "chain900" and "onehot" at -900
        chain = kind.startswith("chain")
        x = np.full((batch, L, V), -30.0 if kind == "chain" else -900.0, np.float32)
        x[:, :, 3] = rng.uniform(-5, 5, (batch, L)).astype(np.float32)
        x[:, ::2, 7] = x[:, ::2, 3] - (5.0 if chain else 0.5)
    return gen.f32_to_bf16_bits(x) if dt == BF16 else x


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
def test_build_edge_cases(case):
    name, L, V, B, dt, kind = case
    _say("edge", name)
    x = _edge_logits(L, V, dt, kind, 3, seed=len(name) if kind != "chain900" else len(name) - 9)
    g = _gpu_build(x, dt, B)
    o = O.build(x, dt, B)
    _check_counts(compare_batch(g, o, B), f"edge {name}")
    _check_mask_of_own_parents(g, B)


def test_build_is_deterministic_and_reuses_workspace():
    # 100 repeats on the batch-64 workload (one cached workspace), every
    # output compared bit for bit with the first call's, on the device
    x = _inputs(3, 1, batch=64)
    d = to_device(x, BF16)
    a = {k: v.clone() for k, v in pkg.ddtree_build(d, 128).items()}
    out = pkg.ddtree_build(d, 128)
    bad = []
    for i in range(100):
        pkg.ddtree_build(d, 128, out=out)
        for k in a:
            if not torch.equal(a[k], out[k]):
                bad.append((i, k))
    assert not bad, bad[:5]


def test_build_rejects_bad_arguments():
    d = to_device(_inputs(1, 0), F32)
    with pytest.raises(pkg.DDTreeError) as e:
        pkg.ddtree_build(d, 1000)
    assert e.value.status == -2
    with pytest.raises(ValueError, match="contiguous"):
        pkg.ddtree_build(d.transpose(1, 2).contiguous().transpose(1, 2), 32)
    t = pkg.ddtree_build(d, 32)
    bad_tgt = torch.zeros((33, 2), dtype=torch.int32, device=DEV).t()[:1]
    with pytest.raises(ValueError, match="contiguous"):
        pkg.ddtree_accept(t["tree_tokens"], t["parents"], t["num_nodes"], bad_tgt, 15)
    with pytest.raises(TypeError):
        pkg.ddtree_accept(t["tree_tokens"], t["parents"], t["num_nodes"],
                          torch.zeros((1, 33), dtype=torch.int64, device=DEV), 15)


# ----------------------------------------------------------------------------
# stages 3 and 4 on oracle trees
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,seed", [(1, 0), (2, 0), (3, 2)])
def test_mask_kernel_on_oracle_trees(cfg, seed):
    B = gen.CONFIGS[cfg]["B"]
    o = _oracle(cfg, seed, batch=min(4, gen.CONFIGS[cfg]["batch"]))
    m = pkg.ddtree_mask(torch.from_numpy(o["parents"]).to(DEV),
                        torch.from_numpy(o["num_nodes"]).to(DEV), B)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(m.cpu().numpy().view(np.uint64),
                                  O.mask(o["parents"], o["num_nodes"], B))


@pytest.mark.parametrize("B", [1, 63, 200, 512])
def test_mask_kernel_random_trees(B):
    """Random prefix-ordered trees (parent of node j+1 drawn from 0..j), deep
    and wide, every row width up to nine words; node counts below B too."""
    rng = np.random.default_rng(B)
    batch = 6
    par = np.full((batch, B), -1, np.int32)
    nn = np.array([B, B, B // 2, 1, 0, max(B - 1, 0)], np.int32)
    for b in range(batch):
        for j in range(nn[b]):
            par[b, j] = j if b == 1 else int(rng.integers(0, j + 1))  # b = 1: one chain
    m = pkg.ddtree_mask(torch.from_numpy(par).to(DEV), torch.from_numpy(nn).to(DEV), B)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(m.cpu().numpy().view(np.uint64), O.mask(par, nn, B))


def _walk_both(o, tgt, L):
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    r = pkg.ddtree_accept(dv(o["tree_tokens"]), dv(o["parents"]), dv(o["num_nodes"]), dv(tgt), L)
    torch.cuda.synchronize()
    ga = [r[k].cpu().numpy() for k in ("accepted_nodes", "accept_len", "next_token")]
    oa = O.accept(o["tree_tokens"], o["parents"], o["num_nodes"], tgt, L)
    for a, b in zip(ga, oa):
        np.testing.assert_array_equal(a, b)
    return ga


def test_walk_c1_fresh_argmax_targets():
    for seed in range(5):
        o = _oracle(1, seed)
        tgt = gen.fresh_argmax_targets(1, seed, 1, 32, 1024)
        _walk_both(o, tgt, 15)


@pytest.mark.parametrize("cfg,seed", [(2, 1), (3, 0)])
def test_walk_drafter_targets_on_oracle_trees(cfg, seed):
    x = _inputs(cfg, seed)
    o = _oracle(cfg, seed)
    B = gen.CONFIGS[cfg]["B"]
    Y = gen.drafter_draws(cfg, seed, x, BF16)
    tgt = gen.node_targets_from_depths(Y, o["depths"], o["num_nodes"], B)
    _, alen, _ = _walk_both(o, tgt, 15)
    _say(f"workload {cfg} accept_len mean", float(alen.mean()))


def test_prop1_monte_carlo_through_gpu_walk():
    # Proposition 1 (DDTree explainer, section 3): E[accepted] = sum_u q(u),
    # with the walk run on the GPU over 2e5 draws Y ~ Q.
    rng = np.random.default_rng(11)
    L, V, B, N = 6, 12, 24, 200000
    x = (rng.uniform(0.5, 2.5) * rng.standard_normal((1, L, V))).astype(np.float32)
    g = _gpu_build(x, F32, B)
    o = O.build(x, F32, B)
    assert classify(g, o, 0, B) == "exact"
    from scipy.special import log_softmax
    p = np.exp(log_softmax(x[0].astype(np.float64), axis=1))
    Y = np.empty((N, L + 1), np.int64)
    for d in range(L):
        Y[:, d] = np.minimum(np.searchsorted(np.cumsum(p[d]), rng.random(N), side="right"), V - 1)
    Y[:, L] = 0
    n = int(g["num_nodes"][0])
    dep = np.concatenate([[0], g["depths"][0]])
    tgt = np.ascontiguousarray(Y[:, dep], dtype=np.int32)
    tgt[:, n + 1:] = 0
    rep = lambda a: torch.from_numpy(np.repeat(a, N, axis=0)).to(DEV)
    r = pkg.ddtree_accept(rep(g["tree_tokens"]), rep(g["parents"]), rep(g["num_nodes"]),
                          torch.from_numpy(tgt).to(DEV), L)
    alen = r["accept_len"].cpu().numpy()
    expected = float(np.exp(o["score64"][0, :n]).sum())
    se = alen.std() / math.sqrt(N)
    assert abs(alen.mean() - expected) < 5 * se


@pytest.mark.parametrize("a,g,printed", [(0.5, 4, 1.94), (0.5, 8, 2.00), (0.8, 4, 3.4)])
def test_chain_closed_form_through_gpu(a, g, printed):
    # DSpark guide page: tokens per pass (1 - a^(g+1)) / (1 - a).
    V = 10 if (a, g) != (0.5, 8) else 256
    row = np.full(V, math.log((1 - a) / (V - 1)))
    row[0] = math.log(a)
    x = np.tile(row.astype(np.float32), (1, g, 1))
    t = _gpu_build(x, F32, g)
    assert list(t["depths"][0]) == list(range(1, g + 1))
    assert list(t["parents"][0]) == list(range(g))
    tokens = 1.0 + float(np.exp(t["logq"][0].astype(np.float64)).sum())
    assert tokens == pytest.approx((1 - a ** (g + 1)) / (1 - a), abs=1e-5)
    assert round(tokens, 2 if printed != 3.4 else 1) == pytest.approx(printed)


def test_build_accept_graph_replays_match_eager():
    # build + accept captured once as a HIP graph; between replays new logits
    # and targets are copied into the captured inputs and the host
    # synchronises; every replay must equal the eager calls on the same input.
    B, L = 64, 15
    xs = [gen.make_logits(2, s) for s in range(3)]
    d = to_device(xs[0], BF16)
    tree = pkg.ddtree_build(d, B)
    tgt = torch.zeros((1, B + 1), dtype=torch.int32, device=DEV)
    acc = pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"], tgt, L)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pkg.ddtree_build(d, B, out=tree)
        pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"], tgt, L, out=acc)
    torch.cuda.synchronize()
    accepted = 0
    for rep in range(6):
        s = rep % 3
        d.copy_(to_device(xs[s], BF16))
        et = to_host(pkg.ddtree_build(d, B))
        Y = gen.drafter_draws(2, s, xs[s], BF16)
        tgt.copy_(torch.from_numpy(gen.node_targets_from_depths(Y, et["depths"], et["num_nodes"], B)))
        ea = to_host(pkg.ddtree_accept(torch.from_numpy(et["tree_tokens"]).to(DEV),
                                       torch.from_numpy(et["parents"]).to(DEV),
                                       torch.from_numpy(et["num_nodes"]).to(DEV), tgt, L))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = to_host({**tree, **acc})
        for k, v in {**et, **ea}.items():
            np.testing.assert_array_equal(got[k], v, err_msg=f"replay {rep}: {k}")
        accepted += int(got["accept_len"][0])
    _say("graph replays: accepted nodes over six rounds", accepted)


def test_two_streams_same_shape_have_separate_workspaces():
    # Few-row builds (the chunk + merge path, which keeps per-chunk records
    # in the workspace) of one shape enqueued on two streams at once: the
    # binding gives each stream its own workspace, so neither call reads the
    # other's records. Both must equal the same builds run alone.
    xs = [_inputs(2, s) for s in (0, 1)]
    ds = [to_device(x, BF16) for x in xs]
    alone = [to_host(pkg.ddtree_build(d, 64)) for d in ds]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for rep in range(3):
        outs = [None, None]
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                outs[i] = pkg.ddtree_build(ds[i], 64)
        torch.cuda.synchronize()
        for i in range(2):
            got = to_host(outs[i])
            for k, v in alone[i].items():
                np.testing.assert_array_equal(got[k], v, err_msg=f"rep {rep} stream {i}: {k}")
    ws_keys = [k for k in pkg._lib._workspaces if k[0] == "build" and k[3][0] == 1]
    assert len({k[2] for k in ws_keys}) >= 2
