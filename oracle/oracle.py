"""ctypes front end of the CPU oracle (``libddtree_oracle.so``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module. It marshals numpy
arrays into the plain-C oracle in ``ddtree_oracle.c`` and adds no arithmetic
of its own. The oracle shares no code with the HIP library.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ddtree_oracle.c")
# DDT_ORACLE_LIB selects another build of the same source (the sanitizer
# build of the CPU checks, see build_oracle(sanitize=True)).
LIB = os.environ.get("DDT_ORACLE_LIB") or os.path.join(HERE, "libddtree_oracle.so")

DTYPE_BF16 = 0
DTYPE_F32 = 1


def build_oracle(sanitize: bool = False, out: str | None = None) -> str:
    """Compile the oracle with gcc -O2 (no fast-math). Returns the library path.

    sanitize=True builds it with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code, gcc; every finding aborts) for the CPU checks that run the pins
    under them; such a library is loaded by a process that preloads libasan.
    """
    out = out or LIB
    flags = ["-O2"]
    if sanitize:
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all"]
    cmd = ["gcc", *flags, "-std=c11", "-fPIC", "-shared", "-o", out + ".tmp", SRC, "-lm",
           "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"oracle library missing: {LIB} (run __graft_entry__.build())")
        L = C.CDLL(LIB)
        p, i32, i64, d = C.c_void_p, C.c_int32, C.c_int64, C.c_double
        L.oracle_row_lse.restype = d
        L.oracle_row_lse.argtypes = [p, C.c_int, i64]
        L.oracle_row_rank.restype = C.c_int
        L.oracle_row_rank.argtypes = [p, C.c_int, i64, i32, p, p]
        L.oracle_select.restype = C.c_int
        L.oracle_select.argtypes = [p, p, p, i32, i32, i32, p, p, p, p, p, p, p, p, p]
        L.oracle_build.restype = C.c_int
        L.oracle_build.argtypes = [p, C.c_int, i64, i32, i64, i32] + [p] * 12 + [C.c_int]
        L.oracle_mask.restype = C.c_int
        L.oracle_mask.argtypes = [p, p, i64, i32, p]
        L.oracle_accept.restype = C.c_int
        L.oracle_accept.argtypes = [p, p, p, p, i64, i32, i32, p, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def row_lse(row: np.ndarray, dtype: int) -> float:
    row = np.ascontiguousarray(row)
    return lib().oracle_row_lse(_ptr(row), dtype, row.shape[-1])


def row_rank(row: np.ndarray, dtype: int, K: int):
    row = np.ascontiguousarray(row)
    ids = np.empty(K, np.int32)
    vals = np.empty(K, np.float64)
    _check(lib().oracle_row_rank(_ptr(row), dtype, row.shape[-1], K, _ptr(ids), _ptr(vals)),
           "row_rank")
    return ids, vals


def select(vals: np.ndarray, ids: np.ndarray, z: np.ndarray, B: int) -> dict:
    """Stage 2 of one request from a sorted top-K table vals/ids [L, K] and z [L]."""
    vals = np.ascontiguousarray(vals, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    z = np.ascontiguousarray(z, np.float64)
    L, K = vals.shape
    out = dict(tree_tokens=np.empty(B, np.int32), parents=np.empty(B, np.int32),
               logq=np.empty(B, np.float32), depths=np.empty(B, np.int32),
               num_nodes=np.empty(1, np.int32), score64=np.empty(B, np.float64),
               next_score=np.empty(1, np.float64), max_heap=np.empty(1, np.int32),
               clamps=np.empty(1, np.int32))
    _check(lib().oracle_select(_ptr(vals), _ptr(ids), _ptr(z), L, K, B,
                               *[_ptr(out[k]) for k in ("tree_tokens", "parents", "logq",
                                                        "depths", "num_nodes", "score64",
                                                        "next_score", "max_heap", "clamps")]),
           "select")
    return out


def build(logits: np.ndarray, dtype: int, B: int, threads: int = 1, tables: bool = True) -> dict:
    """Stages 1+2 over a batch [batch, L, V] of logits (bf16 bits or float32)."""
    logits = np.ascontiguousarray(logits)
    batch, L, V = logits.shape
    K = min(B, V)
    o = dict(tree_tokens=np.empty((batch, B), np.int32), parents=np.empty((batch, B), np.int32),
             logq=np.empty((batch, B), np.float32), depths=np.empty((batch, B), np.int32),
             num_nodes=np.empty(batch, np.int32), score64=np.empty((batch, B), np.float64),
             next_score=np.empty(batch, np.float64), max_heap=np.empty(batch, np.int32),
             clamps=np.empty(batch, np.int32))
    if tables:
        o["z"] = np.empty((batch, L), np.float64)
        o["top_ids"] = np.empty((batch, L, K), np.int32)
        o["top_vals"] = np.empty((batch, L, K), np.float64)
    _check(lib().oracle_build(_ptr(logits), dtype, batch, L, V, B,
                              _ptr(o["tree_tokens"]), _ptr(o["parents"]), _ptr(o["logq"]),
                              _ptr(o["depths"]), _ptr(o["num_nodes"]), _ptr(o["score64"]),
                              _ptr(o["next_score"]), _ptr(o.get("z")), _ptr(o.get("top_ids")),
                              _ptr(o.get("top_vals")), _ptr(o["max_heap"]), _ptr(o["clamps"]),
                              int(threads)), "build")
    return o


def mask(parents: np.ndarray, num_nodes: np.ndarray, B: int) -> np.ndarray:
    parents = np.ascontiguousarray(parents, np.int32)
    num_nodes = np.ascontiguousarray(num_nodes, np.int32)
    batch = num_nodes.shape[0]
    W = (B + 1 + 63) // 64
    m = np.empty((batch, B + 1, W), np.uint64)
    _check(lib().oracle_mask(_ptr(parents), _ptr(num_nodes), batch, B, _ptr(m)), "mask")
    return m


def accept(tree_tokens, parents, num_nodes, target_tokens, L: int):
    tree_tokens = np.ascontiguousarray(tree_tokens, np.int32)
    parents = np.ascontiguousarray(parents, np.int32)
    num_nodes = np.ascontiguousarray(num_nodes, np.int32)
    target_tokens = np.ascontiguousarray(target_tokens, np.int32)
    batch, B = tree_tokens.shape
    acc = np.empty((batch, L), np.int32)
    alen = np.empty(batch, np.int32)
    nxt = np.empty(batch, np.int32)
    _check(lib().oracle_accept(_ptr(tree_tokens), _ptr(parents), _ptr(num_nodes),
                               _ptr(target_tokens), batch, B, L, _ptr(acc), _ptr(alen),
                               _ptr(nxt)), "accept")
    return acc, alen, nxt
