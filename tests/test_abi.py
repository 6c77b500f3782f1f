"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""

from __future__ import annotations

import ctypes as C
import os
import re

import pytest

from draft_tree_construction_depth_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddtree.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from draft_tree_construction_depth_amd import _build
        _build.build_library()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:ddt|ddtree|treespark|sparkling|dspark)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for n in ("ddtree_build", "ddtree_select", "ddtree_mask", "ddtree_accept", "ddtree_row_topk",
              "ddtree_compact_kv", "treespark_expand", "treespark_workspace_size",
              "sparkling_build", "sparkling_build_workspace_size", "dspark_budget",
              "sparkling_beam",
              "ddtree_build_workspace_size", "ddtree_row_topk_workspace_size",
              "ddt_status_string", "ddt_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(L):
    assert L.ddt_abi_version() == 1
    assert _lib.status_string(0) == "ok"
    assert _lib.status_string(-1) == "invalid argument"
    assert _lib.status_string(-2) == "unsupported size"
    assert _lib.status_string(-3) == "workspace too small"
    assert _lib.status_string(-4) == "HIP launch failed"
    assert _lib.status_string(-99) == "unknown status"


def test_workspace_sizes(L):
    s3 = L.ddtree_build_workspace_size(64, 15, 151936, 128, 0)
    assert s3 > 64 * 15 * 128 * 8
    assert L.ddtree_build_workspace_size(0, 15, 151936, 128, 0) == 0
    assert L.ddtree_build_workspace_size(1, 15, 151936, 128, 7) == 0
    assert L.ddtree_row_topk_workspace_size(960, 151936, 128, 0) > 0
    # more rows never need less workspace
    assert L.ddtree_build_workspace_size(256, 15, 151936, 256, 0) >= s3


def test_treespark_workspace_and_limits(L):
    ws = L.treespark_workspace_size
    ws.restype = C.c_size_t
    ws.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32]
    assert ws(32, 7, 151936, 2560, 4, 4, 32) > 0              # the README shape
    assert ws(32, 7, 151936, 8192, 4, 4, 32) > 0              # 2.5 GB tables: 32-bit offsets
    assert ws(32, 7, 151936, 14144, 4, 4, 32) == 0            # V * H * 2 >= 2^32: unsupported
    assert ws(32, 7, 151936, 2500, 4, 4, 32) == 0             # H not a multiple of 64
    assert ws(32, 17, 151936, 2560, 4, 4, 32) == 0            # D > 16
    assert ws(32, 7, 151936, 2560, 9, 4, 32) == 0             # k > 8


FAKE = C.c_void_p(0x100000)      # never dereferenced: every call below fails validation
MISALIGNED = C.c_void_p(0x100004)


def _build(L, logits=FAKE, dtype=0, batch=1, Lr=15, V=1024, B=32, out=FAKE, ws=FAKE,
           ws_bytes=1 << 30):
    return L.ddtree_build(logits, dtype, batch, Lr, V, B, out, out, out, out, out, out, ws,
                          ws_bytes, None)


def test_build_validation(L):
    assert _build(L, logits=None) == -1
    assert _build(L, out=None) == -1
    assert _build(L, ws=None) == -1
    assert _build(L, dtype=5) == -1
    assert _build(L, B=0) == -1
    assert _build(L, Lr=0) == -1
    assert _build(L, V=0) == -1
    assert _build(L, logits=MISALIGNED) == -1
    assert _build(L, B=513) == -2
    assert _build(L, Lr=33) == -2
    assert _build(L, Lr=16, B=512, V=5000) == -2      # L*K over the supported size
    assert _build(L, ws_bytes=16) == -3
    assert _build(L, batch=0) == 0                     # empty batch: nothing to do


def test_select_validation(L):
    sel = lambda vals=FAKE, batch=1, Lr=15, K=128, B=128, out=FAKE: L.ddtree_select(
        vals, FAKE, FAKE, batch, Lr, K, B, out, out, out, out, out, out, None)
    assert sel(vals=None) == -1
    assert sel(out=None) == -1
    assert sel(K=0) == -1
    assert sel(K=600) == -2
    assert sel(Lr=16, K=512, B=512) == -2
    assert sel(batch=0) == 0


def test_mask_accept_topk_validation(L):
    assert L.ddtree_mask(None, FAKE, 1, 32, FAKE, None) == -1
    assert L.ddtree_mask(FAKE, FAKE, 1, 0, FAKE, None) == -1
    assert L.ddtree_mask(FAKE, FAKE, 1, 600, FAKE, None) == -2
    assert L.ddtree_mask(FAKE, FAKE, 0, 32, FAKE, None) == 0
    assert L.ddtree_accept(FAKE, FAKE, FAKE, None, 1, 32, 15, FAKE, FAKE, FAKE, None) == -1
    assert L.ddtree_accept(FAKE, FAKE, FAKE, FAKE, 1, 32, 0, FAKE, FAKE, FAKE, None) == -1
    assert L.ddtree_accept(FAKE, FAKE, FAKE, FAKE, 1, 32, 40, FAKE, FAKE, FAKE, None) == -2
    assert L.ddtree_accept(FAKE, FAKE, FAKE, FAKE, 0, 32, 15, FAKE, FAKE, FAKE, None) == 0
    assert L.ddtree_row_topk(FAKE, 0, 4, 100, 200, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert L.ddtree_row_topk(FAKE, 0, 4, 1000, 600, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -2
    assert L.ddtree_row_topk(FAKE, 0, 4, 1000, 64, FAKE, FAKE, FAKE, FAKE, 8, None) == -3
    assert L.ddtree_row_topk(MISALIGNED, 0, 4, 1000, 64, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                             None) == -1
    assert L.ddtree_row_topk(FAKE, 0, 0, 1000, 64, FAKE, FAKE, FAKE, FAKE, 0, None) == 0


def test_probe_validation(L):
    assert L.ddtree_read_probe(None, 4, 64, FAKE, None) == -1
    assert L.ddtree_read_probe(FAKE, 4, 60, FAKE, None) == -1
    assert L.ddtree_read_probe(FAKE, 0, 64, FAKE, None) == 0
    # W, E, ptok, V, H, variant, sink
    assert L.ddtree_ts_load_probe(None, FAKE, FAKE, 1000, 128, 0, FAKE, None) == -1
    assert L.ddtree_ts_load_probe(FAKE, FAKE, FAKE, 1000, 100, 0, FAKE, None) == -1
    assert L.ddtree_ts_load_probe(FAKE, FAKE, FAKE, 1000, 128, 8, FAKE, None) == -1
    assert L.ddtree_ts_load_probe(FAKE, FAKE, FAKE, 0, 128, 0, FAKE, None) == -1
    assert L.ddtree_ts_load_probe(MISALIGNED, FAKE, FAKE, 1000, 128, 0, FAKE, None) == -1
    assert L.ddtree_ts_load_probe(FAKE, FAKE, FAKE, 1 << 20, 4096, 0, FAKE, None) == -2


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_compact_kv_validation(L):
    """Rejected before any launch (the pointers below are never dereferenced)."""
    f = L.ddtree_compact_kv
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_int64, C.c_int32,
                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]
    def call(k=FAKE, layers=2, batch=3, heads=4, cap=100, row=256, Lw=15, past=FAKE):
        return f(k, FAKE, layers, batch, heads, cap, row, past, FAKE, FAKE, Lw, FAKE, None)
    assert call(row=100) == -2            # not a multiple of 16 bytes
    assert call(row=2048) == -2           # more than 1 KiB per row
    assert call(Lw=33) == -2              # deeper than DDT_MAX_L
    assert call(Lw=0) == -1
    assert call(cap=0) == -1
    assert call(k=MISALIGNED) == -1
    assert call(past=None) == -1
    assert call(layers=0) == 0            # nothing to do


def test_sparkling_validation(L):
    """Sizes and pointers rejected before any launch (pointers never dereferenced)."""
    ws = L.sparkling_build_workspace_size
    assert ws(64, 15, 151936, 128, 256, 64, 0) > 64 * 14 * 128 * 128 * 4   # conditioned rows
    assert ws(64, 15, 151936, 129, 256, 64, 0) == 0      # C > 128
    assert ws(64, 15, 151936, 128, 200, 64, 0) == 0      # R not a multiple of 64
    assert ws(64, 15, 151936, 128, 320, 64, 0) == 0      # R > 256
    assert ws(64, 18, 151936, 128, 256, 64, 0) == 0      # L * ceil(log2 C) > 122
    assert ws(64, 15, 100, 128, 256, 64, 0) == 0         # C > V
    assert ws(1, 1, 1024, 8, 64, 4, 0) > 0               # one row: no conditioned rows

    def call(logits=FAKE, dtype=0, W1=FAKE, batch=2, Lr=15, V=1024, C=128, R=256, B=64, out=FAKE,
             wsp=FAKE, ws_bytes=1 << 34):
        return L.sparkling_build(logits, dtype, W1, FAKE, batch, Lr, V, C, R, B, out, out, out,
                                 out, out, out, wsp, ws_bytes, None)
    assert call(logits=None) == -1
    assert call(W1=None) == -1
    assert call(out=None) == -1
    assert call(wsp=None) == -1
    assert call(W1=MISALIGNED) == -1
    assert call(dtype=3) == -1
    assert call(C=0) == -1
    assert call(C=2000, V=1024) == -1    # C > V
    assert call(C=200) == -2
    assert call(R=96) == -2
    assert call(B=513) == -2
    assert call(Lr=33) == -2
    assert call(ws_bytes=64) == -3
    assert call(batch=0) == 0            # nothing to do


def test_dspark_validation(L):
    def call(conf=FAKE, batch=4, P=5, cost=FAKE, n_cost=100, keep=FAKE, n_keep=FAKE):
        return L.dspark_budget(conf, batch, P, cost, n_cost, keep, None, n_keep, None, None, None)
    assert call(conf=None) == -1
    assert call(cost=None) == -1
    assert call(keep=None) == -1
    assert call(n_keep=None) == -1
    assert call(P=0) == -1
    assert call(batch=-1) == -1
    assert call(n_cost=4) == -1           # the step without guesses is not costed
    assert call(batch=1000, P=5) == -2    # more than 4096 slots
    assert call(batch=0) == 0


def test_sparkling_beam_validation(L):
    f = L.sparkling_beam

    def call(widths=(4,) * 15, budget=0, Lr=15, Cc=128, R=256, batch=2, out=FAKE, wsp=FAKE,
             ws_bytes=1 << 34):
        wa = None if widths is None else (C_int32 * len(widths))(*widths)
        return f(FAKE, 0, FAKE, FAKE, batch, Lr, 1024, Cc, R,
                 None if wa is None else C.cast(wa, C.c_void_p), budget, out, out, out, out, out,
                 out, wsp, ws_bytes, None)
    C_int32 = C.c_int32
    assert call(widths=None) == -1                # no widths and no budget
    assert call(widths=(0,) * 15) == -1          # empty budget
    assert call(widths=(-1,) + (4,) * 14) == -1
    assert call(widths=(65,) + (4,) * 14) == -2  # a width above 64
    assert call(widths=(64,) * 9, Lr=9) == -2    # B = 576 > 512
    assert call(Cc=200) == -2
    assert call(out=None) == -1
    assert call(ws_bytes=64) == -3
    assert call(batch=0) == 0
    # widths given with a budget: the budget must be their sum
    assert call(budget=61) == -1
    assert call(budget=60, batch=0) == 0
    assert call(budget=-1) == -1


def test_sparkling_beam_even_schedule_on_the_host(L):
    """widths == NULL: the library spreads the budget over the depths (the
    remainder on the first ones), validated on the host before any launch."""
    f = L.sparkling_beam

    def call(budget, Lr=15, ws_bytes=1 << 34, batch=2):
        return f(FAKE, 0, FAKE, FAKE, batch, Lr, 1024, 128, 256, None, budget, FAKE, FAKE, FAKE,
                 FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(0) == -1                 # nothing to spread
    assert call(64, batch=0) == 0        # 5 on four depths, 4 on eleven: valid
    assert call(64, ws_bytes=64) == -3   # checked against the workspace of B = 64
    assert call(15 * 65) == -2           # above DDT_MAX_B
    assert call(3 * 65, Lr=3) == -2      # 65 per depth: above the 64 a depth holds
    assert call(512, Lr=8, batch=0) == 0  # exactly 64 per depth


def test_build_noalloc_host_checks(L):
    """ddtree_build_noalloc validates on the host and rejects shapes beyond its
    16 MiB static scratch before touching the device."""
    f = L.ddtree_build_noalloc

    def call(batch=2, Lr=15, V=151936, B=128, out=FAKE, logits=FAKE):
        return f(logits, 0, batch, Lr, V, B, out, out, out, out, out, out, None)
    assert L.ddtree_build_workspace_size(1100, 15, 2048, 512, 0) > 16 << 20
    assert call(batch=1100, V=2048, B=512) == -2
    assert L.ddtree_build_workspace_size(256, 15, 151936, 256, 0) < 16 << 20
    assert call(B=0) == -1
    assert call(out=None) == -1
    assert call(logits=C.c_void_p(0x100008)) == -1   # not 16-byte aligned
    assert call(B=513) == -2
    assert call(batch=0) == 0
