"""Pins of the KV compaction oracle (DDTree explainer, section 5) against
facts fixed independently of it: a hand-worked example, the rows it must not
touch, and the equivalence with an in-place sequential copy (node numbers
increase along a path, so copying in path order never reads a row it has
already overwritten)."""

import numpy as np
import pytest

from oracle import kv as O


def _cache(layers, batch, heads, cap, dh, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 1 << 16, (layers, batch, heads, cap, dh), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (layers, batch, heads, cap, dh), dtype=np.uint16)
    return k, v


def test_hand_worked_example():
    # one layer, one request, one head, dh = 1: row r holds the value 10 r.
    cap = 12
    k = (10 * np.arange(cap, dtype=np.uint16)).reshape(1, 1, 1, cap, 1)
    v = k + 1
    past = np.array([3], np.int32)
    accepted = np.array([[2, 5, 6, -1]], np.int32)  # the path root -> node 2 -> node 5 -> node 6
    k2, v2, n = O.compact(k, v, past, accepted, np.array([3], np.int32))
    # rows 0..3 keep 0..30 (the root sits at row 3), rows 4, 5, 6 take the rows of
    # nodes 2, 5, 6 (rows 5, 8, 9 -> 50, 80, 90), rows 7.. keep their values
    assert k2[0, 0, 0, :, 0].tolist() == [0, 10, 20, 30, 50, 80, 90, 70, 80, 90, 100, 110]
    assert (v2 == k2 + 1).all()
    assert n.tolist() == [7]


def test_nothing_accepted_changes_nothing():
    k, v = _cache(2, 3, 2, 20, 4)
    past = np.array([0, 5, 7], np.int32)
    acc = np.full((3, 4), -1, np.int32)
    k2, v2, n = O.compact(k, v, past, acc, np.zeros(3, np.int32))
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    assert n.tolist() == [1, 6, 8]


@pytest.mark.parametrize("seed", range(4))
def test_rows_outside_the_path_slots_untouched_and_inputs_kept(seed):
    rng = np.random.default_rng(seed)
    layers, batch, heads, cap, dh, B, L = 3, 4, 2, 64, 8, 20, 6
    k, v = _cache(layers, batch, heads, cap, dh, seed)
    k0, v0 = k.copy(), v.copy()
    past = rng.integers(0, cap - B - 1, batch).astype(np.int32)
    n = rng.integers(0, L + 1, batch).astype(np.int32)
    acc = np.full((batch, L), -1, np.int32)
    for b in range(batch):
        acc[b, :n[b]] = np.sort(rng.choice(np.arange(1, B + 1), n[b], replace=False))
    k2, v2, nl = O.compact(k, v, past, acc, n)
    assert np.array_equal(k, k0) and np.array_equal(v, v0)
    for b in range(batch):
        keep = np.ones(cap, bool)
        keep[past[b] + 1: past[b] + n[b] + 1] = False
        assert np.array_equal(k2[:, b][:, :, keep], k[:, b][:, :, keep])
        assert np.array_equal(v2[:, b][:, :, keep], v[:, b][:, :, keep])
        for i in range(1, n[b] + 1):
            assert np.array_equal(k2[:, b, :, past[b] + i], k[:, b, :, past[b] + acc[b, i - 1]])
    assert nl.tolist() == (past + n + 1).tolist()


def test_matches_in_place_sequential_copy():
    """Copying in path order in place gives the same cache: a_i >= i, so the
    source of step i has not been overwritten by steps 1..i-1."""
    rng = np.random.default_rng(7)
    k, v = _cache(2, 5, 3, 80, 4, 7)
    past = rng.integers(0, 40, 5).astype(np.int32)
    L, B = 8, 30
    n = rng.integers(0, L + 1, 5).astype(np.int32)
    acc = np.full((5, L), -1, np.int32)
    for b in range(5):
        acc[b, :n[b]] = np.sort(rng.choice(np.arange(1, B + 1), n[b], replace=False))
    k2, v2, _ = O.compact(k, v, past, acc, n)
    k3, v3 = k.copy(), v.copy()
    for b in range(5):
        for i in range(1, n[b] + 1):
            assert acc[b, i - 1] >= i
            k3[:, b, :, past[b] + i] = k3[:, b, :, past[b] + acc[b, i - 1]]
            v3[:, b, :, past[b] + i] = v3[:, b, :, past[b] + acc[b, i - 1]]
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)
