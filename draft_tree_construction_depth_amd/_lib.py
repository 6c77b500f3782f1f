"""ctypes binding of libddtree.so (C ABI in include/ddtree.h).

Argument marshalling only: every function below passes torch tensors' device
pointers and the current HIP stream to the function of the same name in the
library; all computation happens in the library's HIP kernels. There is no
fallback: if the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libddtree.so")

DDT_OK, DDT_EINVAL, DDT_ENOTSUP, DDT_EWORKSPACE, DDT_EHIP = 0, -1, -2, -3, -4
DDT_BF16, DDT_F32 = 0, 1

_lib = None


class DDTreeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib() -> C.CDLL:
    """Load libddtree.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.ddt_abi_version.restype = C.c_int
        L.ddt_status_string.restype = C.c_char_p
        L.ddt_status_string.argtypes = [C.c_int]
        L.ddtree_build_workspace_size.restype = sz
        L.ddtree_build_workspace_size.argtypes = [i64, i32, i64, i32, C.c_int]
        L.ddtree_row_topk_workspace_size.restype = sz
        L.ddtree_row_topk_workspace_size.argtypes = [i64, i64, i32, C.c_int]
        L.ddtree_build.restype = C.c_int
        L.ddtree_build.argtypes = [p, C.c_int, i64, i32, i64, i32, p, p, p, p, p, p, p, sz, p]
        L.ddtree_build_noalloc.restype = C.c_int
        L.ddtree_build_noalloc.argtypes = [p, C.c_int, i64, i32, i64, i32, p, p, p, p, p, p, p]
        L.ddtree_select.restype = C.c_int
        L.ddtree_select.argtypes = [p, p, p, i64, i32, i32, i32, p, p, p, p, p, p, p]
        L.ddtree_mask.restype = C.c_int
        L.ddtree_mask.argtypes = [p, p, i64, i32, p, p]
        L.ddtree_accept.restype = C.c_int
        L.ddtree_accept.argtypes = [p, p, p, p, i64, i32, i32, p, p, p, p]
        L.ddtree_compact_kv.restype = C.c_int
        L.ddtree_compact_kv.argtypes = [p, p, i64, i64, i32, i64, i32, p, p, p, i32, p, p]
        L.ddtree_read_probe.restype = C.c_int
        L.ddtree_read_probe.argtypes = [p, i64, i64, p, p]
        L.ddtree_ts_load_probe.restype = C.c_int
        L.ddtree_ts_load_probe.argtypes = [p, p, p, i64, i32, i32, p, p]
        L.ddtree_row_topk.restype = C.c_int
        L.ddtree_row_topk.argtypes = [p, C.c_int, i64, i64, i32, p, p, p, p, sz, p]
        L.treespark_workspace_size.restype = sz
        L.treespark_workspace_size.argtypes = [i64, i32, i64, i32, i32, i32, i32]
        L.treespark_expand.restype = C.c_int
        L.treespark_expand.argtypes = [p, p, p, p, i64, i32, i64, i32, i32, i32, i32, p, p, p, p,
                                       p, p, sz, p]
        L.sparkling_build_workspace_size.restype = sz
        L.sparkling_build_workspace_size.argtypes = [i64, i32, i64, i32, i32, i32, C.c_int]
        L.sparkling_build.restype = C.c_int
        L.sparkling_build.argtypes = [p, C.c_int, p, p, i64, i32, i64, i32, i32, i32, p, p, p, p,
                                      p, p, p, sz, p]
        L.dspark_budget.restype = C.c_int
        L.dspark_budget.argtypes = [p, i64, i32, p, i32, p, p, p, p, p, p]
        L.sparkling_beam.restype = C.c_int
        L.sparkling_beam.argtypes = [p, C.c_int, p, p, i64, i32, i64, i32, i32, p, i32, p, p, p,
                                     p, p, p, p, sz, p]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ddt_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _arg(t, name, dtypes, shape=None):
    """Check that a tensor argument is a contiguous device tensor of the
    expected dtype (and shape); the library reads raw row-major memory."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


_I32 = (torch.int32,)
_LOGITS = (torch.bfloat16, torch.float32)


def _stream(device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DDT_BF16
    if t.dtype == torch.float32:
        return DDT_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _check(fn, rc):
    if rc != DDT_OK:
        raise DDTreeError(fn, rc)


_workspaces: dict = {}


def workspace(kind: str, size: int, device, key) -> torch.Tensor:
    """Scratch buffer cached per (kind, device, stream, shape key).

    The library ignores a workspace's contents on entry, so one buffer per
    shape is reused across calls; calls on different streams may overlap and
    so get buffers of their own.
    """
    k = (kind, str(device), torch.cuda.current_stream(device).cuda_stream, key)
    ws = _workspaces.get(k)
    if ws is None or ws.numel() < size:
        ws = torch.empty(max(size, 1), dtype=torch.uint8, device=device)
        _workspaces[k] = ws
    return ws


def ddtree_build(logits: torch.Tensor, B: int, *, with_mask: bool = True, out: dict | None = None,
                 ws: torch.Tensor | None = None) -> dict:
    """Stages 1-2 (+3): logits [batch, L, V] (bf16/f32, cuda) -> tree tensors."""
    _arg(logits, "logits", _LOGITS)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, L, V]")
    batch, L, V = logits.shape
    dev = logits.device
    dt = _dtype_code(logits)
    if out is None:
        out = _tree_out(batch, B, dev, with_mask)
    size = lib().ddtree_build_workspace_size(batch, L, V, B, dt)
    if ws is None:
        ws = workspace("build", size, dev, (batch, L, V, B, dt))
    rc = lib().ddtree_build(_ptr(logits), dt, batch, L, V, B, _ptr(out["tree_tokens"]),
                            _ptr(out["parents"]), _ptr(out["logq"]), _ptr(out.get("depths")),
                            _ptr(out["num_nodes"]), _ptr(out.get("mask")), _ptr(ws),
                            ws.numel(), _stream(dev))
    _check("ddtree_build", rc)
    return out


def ddtree_build_noalloc(logits: torch.Tensor, B: int, *, with_mask: bool = True,
                         out: dict | None = None) -> dict:
    """ddtree_build on the library's static scratch (no workspace; the call
    allocates nothing on the device when out is given)."""
    _arg(logits, "logits", _LOGITS)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, L, V]")
    batch, L, V = logits.shape
    dev = logits.device
    dt = _dtype_code(logits)
    if out is None:
        out = _tree_out(batch, B, dev, with_mask)
    rc = lib().ddtree_build_noalloc(_ptr(logits), dt, batch, L, V, B, _ptr(out["tree_tokens"]),
                                    _ptr(out["parents"]), _ptr(out["logq"]),
                                    _ptr(out.get("depths")), _ptr(out["num_nodes"]),
                                    _ptr(out.get("mask")), _stream(dev))
    _check("ddtree_build_noalloc", rc)
    return out


def _tree_out(batch, B, dev, with_mask):
    out = dict(
        tree_tokens=torch.empty((batch, B), dtype=torch.int32, device=dev),
        parents=torch.empty((batch, B), dtype=torch.int32, device=dev),
        logq=torch.empty((batch, B), dtype=torch.float32, device=dev),
        depths=torch.empty((batch, B), dtype=torch.int32, device=dev),
        num_nodes=torch.empty((batch,), dtype=torch.int32, device=dev),
    )
    if with_mask:
        out["mask"] = torch.empty((batch, B + 1, (B + 1 + 63) // 64), dtype=torch.int64, device=dev)
    return out


def ddtree_select(vals: torch.Tensor, ids: torch.Tensor, lse: torch.Tensor, B: int, *,
                  with_mask: bool = True, out: dict | None = None) -> dict:
    """Stage 2 (+3) from tables vals/ids [batch, L, K] and lse [batch, L]."""
    _arg(vals, "vals", (torch.float32,))
    batch, L, K = vals.shape
    _arg(ids, "ids", _I32, (batch, L, K))
    _arg(lse, "lse", (torch.float64,), (batch, L))
    if out is None:
        out = _tree_out(batch, B, vals.device, with_mask)
    rc = lib().ddtree_select(_ptr(vals), _ptr(ids), _ptr(lse), batch, L, K, B,
                             _ptr(out["tree_tokens"]), _ptr(out["parents"]), _ptr(out["logq"]),
                             _ptr(out.get("depths")), _ptr(out["num_nodes"]), _ptr(out.get("mask")),
                             _stream(vals.device))
    _check("ddtree_select", rc)
    return out


def ddtree_mask(parents: torch.Tensor, num_nodes: torch.Tensor, B: int,
                mask: torch.Tensor | None = None) -> torch.Tensor:
    _arg(num_nodes, "num_nodes", _I32)
    batch = num_nodes.shape[0]
    _arg(parents, "parents", _I32, (batch, B))
    W = (B + 1 + 63) // 64
    if mask is None:
        mask = torch.empty((batch, B + 1, W), dtype=torch.int64, device=parents.device)
    rc = lib().ddtree_mask(_ptr(parents), _ptr(num_nodes), batch, B, _ptr(mask),
                           _stream(parents.device))
    _check("ddtree_mask", rc)
    return mask


def ddtree_accept(tree_tokens: torch.Tensor, parents: torch.Tensor, num_nodes: torch.Tensor,
                  target_tokens: torch.Tensor, L: int, out: dict | None = None) -> dict:
    _arg(tree_tokens, "tree_tokens", _I32)
    batch, B = tree_tokens.shape
    _arg(parents, "parents", _I32, (batch, B))
    _arg(num_nodes, "num_nodes", _I32, (batch,))
    _arg(target_tokens, "target_tokens", _I32, (batch, B + 1))
    dev = tree_tokens.device
    if out is None:
        out = dict(accepted_nodes=torch.empty((batch, L), dtype=torch.int32, device=dev),
                   accept_len=torch.empty((batch,), dtype=torch.int32, device=dev),
                   next_token=torch.empty((batch,), dtype=torch.int32, device=dev))
    rc = lib().ddtree_accept(_ptr(tree_tokens), _ptr(parents), _ptr(num_nodes),
                             _ptr(target_tokens), batch, B, L, _ptr(out["accepted_nodes"]),
                             _ptr(out["accept_len"]), _ptr(out["next_token"]), _stream(dev))
    _check("ddtree_accept", rc)
    return out


def ddtree_compact_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, past_len: torch.Tensor,
                      accepted_nodes: torch.Tensor, accept_len: torch.Tensor,
                      new_len: torch.Tensor | None = None) -> torch.Tensor:
    """In place: caches [layers, batch, heads, cap, head_dim] keep the accepted path's
    rows (slots past_len+1 .. past_len+accept_len); returns new_len [batch]."""
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 5:
        raise ValueError("k_cache must be a 5-d tensor [layers, batch, heads, cap, head_dim]")
    _arg(k_cache, "k_cache", (k_cache.dtype,))
    _arg(v_cache, "v_cache", (k_cache.dtype,), tuple(k_cache.shape))
    layers, batch, heads, cap, dh = k_cache.shape
    _arg(past_len, "past_len", _I32, (batch,))
    _arg(accepted_nodes, "accepted_nodes", _I32)
    L = accepted_nodes.shape[-1]
    _arg(accepted_nodes, "accepted_nodes", _I32, (batch, L))
    _arg(accept_len, "accept_len", _I32, (batch,))
    dev = k_cache.device
    if new_len is None:
        new_len = torch.empty((batch,), dtype=torch.int32, device=dev)
    rc = lib().ddtree_compact_kv(_ptr(k_cache), _ptr(v_cache), layers, batch, heads, cap,
                                 dh * k_cache.element_size(), _ptr(past_len),
                                 _ptr(accepted_nodes), _ptr(accept_len), L, _ptr(new_len),
                                 _stream(dev))
    _check("ddtree_compact_kv", rc)
    return new_len


def ddtree_row_topk(logits: torch.Tensor, K: int, *, out: dict | None = None,
                    ws: torch.Tensor | None = None) -> dict:
    """Stage 1 alone: logits [..., V] -> ids/vals [rows, K], lse [rows] (float64)."""
    _arg(logits, "logits", _LOGITS)
    V = logits.shape[-1]
    rows = logits.numel() // V
    dev = logits.device
    dt = _dtype_code(logits)
    if out is None:
        out = dict(ids=torch.empty((rows, K), dtype=torch.int32, device=dev),
                   vals=torch.empty((rows, K), dtype=torch.float32, device=dev),
                   lse=torch.empty((rows,), dtype=torch.float64, device=dev))
    size = lib().ddtree_row_topk_workspace_size(rows, V, K, dt)
    if ws is None:
        ws = workspace("row_topk", size, dev, (rows, V, K, dt))
    rc = lib().ddtree_row_topk(_ptr(logits), dt, rows, V, K, _ptr(out["ids"]), _ptr(out["vals"]),
                               _ptr(out["lse"]), _ptr(ws), ws.numel(), _stream(dev))
    _check("ddtree_row_topk", rc)
    return out


_BF16 = (torch.bfloat16,)


def ddtree_read_probe(src: torch.Tensor, rows: int, row_bytes: int,
                      sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement probe: stream rows x row_bytes bytes of src (stage 1's
    launch geometry, no compute); returns the XOR sink [rows, 4] (uint32 as int32)."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    if rows * row_bytes > src.numel() * src.element_size():
        raise ValueError("rows x row_bytes exceeds src")
    if sink is None:
        sink = torch.empty((rows, 4), dtype=torch.int32, device=src.device)
    _check("ddtree_read_probe", lib().ddtree_read_probe(_ptr(src), rows, row_bytes, _ptr(sink),
                                                        _stream(src.device)))
    return sink


def ddtree_ts_load_probe(W: torch.Tensor, E: torch.Tensor, ptok: torch.Tensor, variant: int,
                         sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement probe: one TreeSpark head evaluation's loads (W [V, H] and
    the 128 parents' rows ptok of E [V, H], bf16) with nothing computed;
    variant 0-4 as in the header. Returns the sink [256] (int32)."""
    _arg(W, "W", _BF16)
    V, H = W.shape
    _arg(E, "E", _BF16, (V, H))
    _arg(ptok, "ptok", _I32, (128,))
    if sink is None:
        sink = torch.empty(256, dtype=torch.int32, device=W.device)
    _check("ddtree_ts_load_probe", lib().ddtree_ts_load_probe(_ptr(W), _ptr(E), _ptr(ptok), V, H,
                                                              variant, _ptr(sink),
                                                              _stream(W.device)))
    return sink


def treespark_expand(backbone: torch.Tensor, W: torch.Tensor, E: torch.Tensor,
                     anchor: torch.Tensor, *, k: int = 4, F: int = 4, N: int = 32,
                     out: dict | None = None, ws: torch.Tensor | None = None) -> dict:
    """TreeSpark expansion: backbone [batch, D, V], W / E [V, H] (bf16), anchor [batch]."""
    _arg(backbone, "backbone", _BF16)
    batch, D, V = backbone.shape
    _arg(W, "W", _BF16)
    Vw, H = W.shape
    if Vw != V:
        raise ValueError(f"W must have {V} rows, got {Vw}")
    _arg(E, "E", _BF16, (V, H))
    _arg(anchor, "anchor", _I32, (batch,))
    dev = backbone.device
    if out is None:
        out = dict(tree_tokens=torch.empty((batch, N), dtype=torch.int32, device=dev),
                   parents=torch.empty((batch, N), dtype=torch.int32, device=dev),
                   logq=torch.empty((batch, N), dtype=torch.float32, device=dev),
                   depths=torch.empty((batch, N), dtype=torch.int32, device=dev),
                   num_nodes=torch.empty((batch,), dtype=torch.int32, device=dev))
    size = lib().treespark_workspace_size(batch, D, V, H, k, F, N)
    if ws is None:
        ws = workspace("treespark", size, dev, (batch, D, V, H, k, F, N))
    rc = lib().treespark_expand(_ptr(backbone), _ptr(W), _ptr(E), _ptr(anchor), batch, D, V, H, k,
                                F, N, _ptr(out["tree_tokens"]), _ptr(out["parents"]),
                                _ptr(out["logq"]), _ptr(out.get("depths")),
                                _ptr(out["num_nodes"]), _ptr(ws), ws.numel(), _stream(dev))
    _check("treespark_expand", rc)
    return out


def sparkling_build(logits: torch.Tensor, W1: torch.Tensor, W2t: torch.Tensor, B: int, *,
                    C: int = 128, with_mask: bool = True, out: dict | None = None,
                    ws: torch.Tensor | None = None) -> dict:
    """SparklingTree: logits [batch, L, V] (bf16/f32), Markov head W1 / W2t [V, R] (bf16)
    -> tree tensors (as ddtree_build)."""
    _arg(logits, "logits", _LOGITS)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, L, V]")
    batch, L, V = logits.shape
    _arg(W1, "W1", _BF16)
    if W1.dim() != 2 or W1.shape[0] != V:
        raise ValueError(f"W1 must be [{V}, R]")
    R = W1.shape[1]
    _arg(W2t, "W2t", _BF16, (V, R))
    dev = logits.device
    dt = _dtype_code(logits)
    if out is None:
        out = _tree_out(batch, B, dev, with_mask)
    size = lib().sparkling_build_workspace_size(batch, L, V, C, R, B, dt)
    if ws is None:
        ws = workspace("sparkling", size, dev, (batch, L, V, C, R, B, dt))
    rc = lib().sparkling_build(_ptr(logits), dt, _ptr(W1), _ptr(W2t), batch, L, V, C, R, B,
                               _ptr(out["tree_tokens"]), _ptr(out["parents"]), _ptr(out["logq"]),
                               _ptr(out.get("depths")), _ptr(out["num_nodes"]),
                               _ptr(out.get("mask")), _ptr(ws), ws.numel(), _stream(dev))
    _check("sparkling_build", rc)
    return out


def dspark_budget(conf: torch.Tensor, cost_ms: torch.Tensor, *, out: dict | None = None) -> dict:
    """DSpark budget: conf [batch, P] float32, cost_ms [n_cost] float32 (cuda) ->
    keep [batch], n_keep [1], survival [batch, P], expected_tokens [1], objective [1]."""
    _arg(conf, "conf", (torch.float32,))
    if conf.dim() != 2:
        raise ValueError("conf must be [batch, P]")
    _arg(cost_ms, "cost_ms", (torch.float32,))
    if cost_ms.dim() != 1:
        raise ValueError("cost_ms must be 1-D")
    batch, P = conf.shape
    dev = conf.device
    if out is None:
        out = dict(keep=torch.empty((batch,), dtype=torch.int32, device=dev),
                   n_keep=torch.empty((1,), dtype=torch.int32, device=dev),
                   survival=torch.empty((batch, P), dtype=torch.float64, device=dev),
                   expected_tokens=torch.empty((1,), dtype=torch.float64, device=dev),
                   objective=torch.empty((1,), dtype=torch.float64, device=dev))
    rc = lib().dspark_budget(_ptr(conf), batch, P, _ptr(cost_ms), cost_ms.numel(),
                             _ptr(out["keep"]), _ptr(out.get("survival")), _ptr(out["n_keep"]),
                             _ptr(out.get("expected_tokens")), _ptr(out.get("objective")),
                             _stream(dev))
    _check("dspark_budget", rc)
    return out


def sparkling_beam(logits: torch.Tensor, W1: torch.Tensor, W2t: torch.Tensor, widths=None, *,
                   B: int | None = None, C: int = 128, with_mask: bool = True,
                   out: dict | None = None, ws: torch.Tensor | None = None) -> dict:
    """Beam tree on SparklingTree's rows: per-depth widths, or (widths None) the
    budget B spread evenly by the library."""
    _arg(logits, "logits", _LOGITS)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, L, V]")
    batch, L, V = logits.shape
    _arg(W1, "W1", _BF16)
    if W1.dim() != 2 or W1.shape[0] != V:
        raise ValueError(f"W1 must be [{V}, R]")
    R = W1.shape[1]
    _arg(W2t, "W2t", _BF16, (V, R))
    import ctypes  # (the argument C shadows the module alias)
    if widths is None:
        if B is None:
            raise ValueError("give widths or a budget B")
        Bt, wa = int(B), None
    else:
        widths = [int(w) for w in widths]
        if len(widths) != L:
            raise ValueError(f"widths must have {L} entries")
        Bt = sum(widths)
        wa = ctypes.cast((ctypes.c_int32 * L)(*widths), ctypes.c_void_p)
    dev = logits.device
    dt = _dtype_code(logits)
    if out is None:
        out = _tree_out(batch, max(Bt, 1), dev, with_mask)
    size = lib().sparkling_build_workspace_size(batch, L, V, C, R, max(Bt, 1), dt)
    if ws is None:
        ws = workspace("sparkling", size, dev, (batch, L, V, C, R, max(Bt, 1), dt))
    rc = lib().sparkling_beam(_ptr(logits), dt, _ptr(W1), _ptr(W2t), batch, L, V, C, R, wa,
                              0 if widths is not None else Bt,
                              _ptr(out["tree_tokens"]), _ptr(out["parents"]), _ptr(out["logq"]),
                              _ptr(out.get("depths")), _ptr(out["num_nodes"]),
                              _ptr(out.get("mask")), _ptr(ws), ws.numel(), _stream(dev))
    _check("sparkling_beam", rc)
    return out
