"""GPU parity of ddtree_compact_kv (DDTree explainer, section 5, KV cache
management) against the CPU oracle: bit-exact caches and new lengths."""

import numpy as np
import pytest
import torch

import draft_tree_construction_depth_amd as pkg
from draft_tree_construction_depth_amd import gen
from oracle import kv as O
from oracle import oracle as OR

pytestmark = pytest.mark.gpu


def _paths(rng, batch, L, B, tight=False):
    """Accepted paths: increasing node numbers with a_i >= i. tight: a_i = i up to a
    random point and i + 1 after it, so a destination row is the next row's source."""
    n = rng.integers(0, L + 1, batch).astype(np.int32)
    acc = np.full((batch, L), -1, np.int32)
    for b in range(batch):
        i = np.arange(1, n[b] + 1)
        if tight:
            m = rng.integers(1, n[b] + 2)
            acc[b, :n[b]] = i + (i >= m)
        else:
            acc[b, :n[b]] = np.sort(rng.choice(np.arange(1, B + 1), n[b], replace=False))
    return acc, n


def _run(k, v, past, acc, n):
    dev = "cuda"
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    nl = pkg.ddtree_compact_kv(kd, vd, torch.from_numpy(past).to(dev), torch.from_numpy(acc).to(dev),
                               torch.from_numpy(n).to(dev))
    torch.cuda.synchronize()
    return kd.cpu().numpy(), vd.cpu().numpy(), nl.cpu().numpy()


CASES = [
    # layers, batch, heads, cap, dh, dtype, L, B, tight
    (3, 5, 4, 100, 128, np.int16, 15, 64, False),    # 256-byte rows (bf16, head dim 128)
    (2, 3, 2, 64, 64, np.float32, 15, 40, False),    # 256-byte rows of float32
    (1, 2, 1, 300, 512, np.int16, 32, 255, False),   # 1 KiB rows: one row per load instruction
    (2, 4, 3, 50, 8, np.int16, 32, 40, False),       # 16-byte rows: 64 rows per instruction
    (2, 6, 2, 80, 128, np.int16, 15, 30, True),      # sources overlapping destinations
    (4, 7, 8, 200, 64, np.int16, 32, 128, False),    # several load batches per wave
]


@pytest.mark.parametrize("seed,case", list(enumerate(CASES)),
                         ids=[f"l{c[0]}b{c[1]}h{c[2]}cap{c[3]}dh{c[4]}{np.dtype(c[5]).name}L{c[6]}"
                              f"{'tight' if c[8] else ''}" for c in CASES])
def test_compact_kv_matches_oracle(seed, case):
    layers, batch, heads, cap, dh, dt, L, B, tight = case
    rng = np.random.default_rng(seed)
    shape = (layers, batch, heads, cap, dh)
    k = rng.integers(-30000, 30000, shape).astype(dt)
    v = rng.integers(-30000, 30000, shape).astype(dt)
    past = rng.integers(0, cap - B - 1, batch).astype(np.int32)
    acc, n = _paths(rng, batch, L, B, tight=tight)
    ko, vo, nlo = O.compact(k, v, past, acc, n)
    kg, vg, nlg = _run(k, v, past, acc, n)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo)
    assert np.array_equal(nlg, nlo)


def test_compact_kv_nothing_accepted():
    rng = np.random.default_rng(3)
    k = rng.integers(-100, 100, (2, 3, 2, 40, 64)).astype(np.int16)
    v = k + 1
    past = np.array([0, 5, 10], np.int32)
    kg, vg, nl = _run(k, v, past, np.full((3, 15), -1, np.int32), np.zeros(3, np.int32))
    assert np.array_equal(kg, k) and np.array_equal(vg, v)
    assert nl.tolist() == [1, 6, 11]


def test_compact_kv_on_walked_paths():
    """Paths from a real build + walk (batch-64 workload shape, 4 requests)."""
    c = gen.CONFIGS[3]
    x = gen.make_logits(3, 2, batch=4)
    o = OR.build(x, c["dtype"], c["B"], threads=4)
    Y = gen.drafter_draws(3, 2, x, c["dtype"])
    tgt = gen.node_targets_from_depths(Y, o["depths"], o["num_nodes"], c["B"])
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    acc = pkg.ddtree_accept(t(o["tree_tokens"]), t(o["parents"]), t(o["num_nodes"]), t(tgt), c["L"])
    torch.cuda.synchronize()
    A, N = acc["accepted_nodes"].cpu().numpy(), acc["accept_len"].cpu().numpy()
    assert N.max() > 0
    rng = np.random.default_rng(5)
    k = rng.integers(-30000, 30000, (3, 4, 2, 400, 128)).astype(np.int16)
    v = rng.integers(-30000, 30000, (3, 4, 2, 400, 128)).astype(np.int16)
    past = np.array([0, 17, 100, 250], np.int32)
    ko, vo, nlo = O.compact(k, v, past, A, N)
    kg, vg, nlg = _run(k, v, past, A, N)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo) and np.array_equal(nlg, nlo)
