"""Python binding of the KPool-DSA sparse-attention library (libkpool.so, C ABI in include/kpool.h).

Argument marshalling only: every stage runs in the library's HIP kernels for gfx950.  torch supplies device
memory and the current stream; nothing else.  There is no fallback: if libkpool.so is missing or fails to load,
every call raises.

The four calls keep the C names:
    kpool_compress, dsa_indexer_score, dsa_topk_select, sparse_mla_attn (sparse_mla_attn_fp8 over an fp8 latent cache)
plus the workspace queries dsa_topk_workspace_size and sparse_mla_workspace_size.  Outputs and workspaces are
caller-allocated tensors, as in the C ABI.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkpool.so")

KP_OK, KP_ERR_INVALID_ARG, KP_ERR_UNSUPPORTED, KP_ERR_WORKSPACE, KP_ERR_LAUNCH = 0, -1, -2, -3, -4
KP_DTYPE_F32, KP_DTYPE_BF16 = 0, 1
ABI_VERSION = 7

EXPORTED = ("kpool_compress", "dsa_indexer_score", "dsa_compress_score", "dsa_topk_workspace_size", "dsa_topk_select",
            "sparse_mla_workspace_size", "sparse_mla_attn", "sparse_mla_attn_shared", "sparse_mla_attn_fp8",
            "sparse_mla_attn_noalloc", "sparse_mla_mtp_workspace_size", "sparse_mla_attn_mtp", "kp_read_rows",
            "kp_linear", "kp_linear_workspace_size", "kp_linear_group", "kp_linear_group_workspace_size",
            "kp_last_error", "kp_abi_version")


class KpError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed ({status}): {msg}")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("heads", ctypes.c_int32), ("latent_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class _Cache(ctypes.Structure):
    _fields_ = [("latent", ctypes.c_void_p), ("pooled", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("bt_stride", ctypes.c_int32)]


class _LinearProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("stride_a", ctypes.c_int64),
                ("W", ctypes.c_void_p), ("ldw", ctypes.c_int64), ("stride_w", ctypes.c_int64),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("stride_c", ctypes.c_int64),
                ("c_dtype", ctypes.c_int32), ("alpha", ctypes.c_float)]


class _Queries(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("seq", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("max_pos", ctypes.c_int32), ("group", ctypes.c_int32)]


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libkpool.so (once).  Raises if it is missing: there is no other implementation."""
    global _lib
    if _lib is not None:
        return _lib
    # torch's HIP runtime first: the library then binds to that same runtime (a process that loaded ROCm's own
    # copy first would hold two, and kernels launched through one would see no device of the other)
    import torch  # noqa: F401
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m sparse_attention_kpool_amd.build` "
                           "(the KPool-DSA layer has no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D, C, Q = ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.POINTER(_Queries)
    lib.kpool_compress.argtypes = [D, C, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.dsa_indexer_score.argtypes = [D, C, Q, vp, vp, vp, i64, vp]
    lib.dsa_compress_score.argtypes = [D, C, i32, vp, vp, vp, vp, vp, vp, Q, vp, vp, vp, i64, vp]
    lib.dsa_topk_workspace_size.argtypes = [D, Q]
    lib.dsa_topk_workspace_size.restype = sz
    lib.dsa_topk_select.argtypes = [D, Q, vp, i64, vp, vp, vp, sz, vp]
    lib.sparse_mla_workspace_size.argtypes = [D, Q]
    lib.sparse_mla_workspace_size.restype = sz
    lib.sparse_mla_attn.argtypes = [D, C, Q, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_mla_attn_fp8.argtypes = [D, C, Q, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.sparse_mla_attn_shared.argtypes = [D, C, Q, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_mla_attn_noalloc.argtypes = [D, C, Q, vp, vp, vp, vp, vp, vp]
    lib.sparse_mla_mtp_workspace_size.argtypes = [D, Q]
    lib.sparse_mla_mtp_workspace_size.restype = sz
    lib.sparse_mla_attn_mtp.argtypes = [D, C, Q, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kp_read_rows.argtypes = [vp, i64, i32, vp, i64, i32, vp]
    lib.kp_linear.argtypes = [i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, vp, i64, i64, i32, ctypes.c_float,
                              vp, sz, vp]
    lib.kp_linear_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.kp_linear_workspace_size.restype = sz
    LP = ctypes.POINTER(_LinearProblem)
    lib.kp_linear_group.argtypes = [i32, LP, vp, sz, vp]
    lib.kp_linear_group_workspace_size.argtypes = [i32, LP]
    lib.kp_linear_group_workspace_size.restype = sz
    for f in ("kpool_compress", "dsa_indexer_score", "dsa_compress_score", "dsa_topk_select", "sparse_mla_attn",
              "sparse_mla_attn_shared",
              "sparse_mla_attn_fp8", "sparse_mla_attn_noalloc", "sparse_mla_attn_mtp", "kp_read_rows", "kp_linear",
              "kp_linear_group"):
        getattr(lib, f).restype = ctypes.c_int
    lib.kp_last_error.restype = ctypes.c_char_p
    lib.kp_abi_version.restype = i32
    if lib.kp_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libkpool.so ABI {lib.kp_abi_version()} != binding ABI {ABI_VERSION}; rebuild")
    _lib = lib
    return lib


def last_error() -> str:
    return load().kp_last_error().decode()


# ----------------------------------------------------------------------------------------------------------
# Python-side descriptions of the C structs
# ----------------------------------------------------------------------------------------------------------
@dataclass
class Dims:
    pool: int = 4
    idx_dim: int = 128
    idx_heads: int = 32
    topk: int = 2048
    heads: int = 64
    latent_dim: int = 576
    v_dim: int = 512
    page_tokens: int = 64
    dtype: str = "bf16"          # 'bf16' or 'f32'
    scale: float = 1.0 / 16.0

    def c(self) -> _Dims:
        return _Dims(self.pool, self.idx_dim, self.idx_heads, self.topk, self.heads, self.latent_dim, self.v_dim,
                     self.page_tokens, KP_DTYPE_BF16 if self.dtype == "bf16" else KP_DTYPE_F32, self.scale)


@dataclass
class Cache:
    latent: object = None        # torch tensor [n_pages, page_tokens, L] (uint8: E4M3 codes, see latent_scale)
    pooled: object = None        # torch tensor [n_pages, page_tokens / P, D]
    block_table: object = None   # torch int32 tensor [n_seq, stride]
    latent_scale: float = 1.0    # scale of an fp8 latent cache (row value = decoded code * latent_scale)

    def c(self) -> _Cache:
        return _Cache(_ptr(self.latent), _ptr(self.pooled), _ptr(self.block_table),
                      int(self.block_table.shape[1]) if self.block_table is not None else 0)


@dataclass
class Queries:
    seq: object                  # torch int32 [n_q]
    pos: object                  # torch int32 [n_q]
    max_pos: int                 # host upper bound of pos
    group: int = 1               # runs of `group` consecutive queries share a sequence (a hint)

    def c(self) -> _Queries:
        return _Queries(int(self.seq.numel()), _ptr(self.seq), _ptr(self.pos), int(self.max_pos), int(self.group))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _check(fn: str, status: int) -> None:
    if status != KP_OK:
        raise KpError(fn, status, last_error())


def _want(fn: str, name: str, t, dtypes, shape, rows_only: bool = False, min_rows: bool = False):
    """Raise ValueError unless `t` is a device tensor of one of `dtypes` with `shape` (None = any extent; with
    min_rows the first extent is a lower bound: the kernels touch rows below it only) that the kernels can address
    densely: contiguous, or (rows_only) a 2-D view whose rows are contiguous."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{fn}: {name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{fn}: {name} must be on the GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    bad = len(shape) != t.dim()
    for d, (e, a) in enumerate(zip(shape, t.shape)):
        if e is not None and (a < e if (min_rows and d == 0) else a != e):
            bad = True
    if bad:
        want = "[" + ", ".join("*" if e is None else (f">={e}" if min_rows and d == 0 else str(e))
                               for d, e in enumerate(shape)) + "]"
        raise ValueError(f"{fn}: {name} has shape {list(t.shape)}, expected {want}")
    if rows_only:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
            raise ValueError(f"{fn}: {name} needs contiguous rows")
    elif not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    return t


def _storage(dims: "Dims"):
    import torch
    return (torch.bfloat16,) if dims.dtype == "bf16" else (torch.float32,)


def _i32():
    import torch
    return (torch.int32,)


def _check_queries(fn: str, queries: "Queries") -> int:
    n = int(queries.seq.numel())
    _want(fn, "queries.seq", queries.seq, _i32(), (n,))
    _want(fn, "queries.pos", queries.pos, _i32(), (n,))
    return n


# ----------------------------------------------------------------------------------------------------------
# the four calls
# ----------------------------------------------------------------------------------------------------------
def _compress_args(fn, dims: Dims, cache: Cache, keys, gates, ape, pool_seq, pool_id, src) -> int:
    """Checks kpool_compress's tensors; returns n_pools."""
    n = int(pool_seq.numel())
    st = _storage(dims)
    _want(fn, "pool_seq", pool_seq, _i32(), (n,))
    _want(fn, "pool_id", pool_id, _i32(), (n,))
    _want(fn, "cache.pooled", cache.pooled, st, (None, dims.page_tokens // dims.pool, dims.idx_dim))
    if n:
        _want(fn, "keys", keys, st, (None, dims.pool, dims.idx_dim))
        if gates is not None:
            _want(fn, "gates", gates, st, tuple(keys.shape))
        if ape is not None:
            _want(fn, "ape", ape, st, (dims.pool, dims.idx_dim))
        if src is not None:
            _want(fn, "src", src, _i32(), (n,))
        elif keys.shape[0] < n:
            raise ValueError(f"{fn}: keys holds {keys.shape[0]} pools, fewer than the {n} to compress")
    return n


def _score_args(fn, dims: Dims, cache: Cache, queries: Queries, q_idx, w, scores) -> None:
    import torch
    n = _check_queries(fn, queries)
    _want(fn, "q_idx", q_idx, _storage(dims), (n, dims.idx_heads, dims.idx_dim), min_rows=True)
    _want(fn, "w", w, (torch.float32,), (n, dims.idx_heads), min_rows=True)
    _want(fn, "scores", scores, (torch.float32,), (n, None), rows_only=True, min_rows=True)
    _want(fn, "cache.pooled", cache.pooled, _storage(dims), (None, dims.page_tokens // dims.pool, dims.idx_dim))


def kpool_compress(dims: Dims, cache: Cache, keys, gates, ape, pool_seq, pool_id, src=None, stream=None) -> None:
    """Pooled keys of complete pools -> rows (pool_seq[i], pool_id[i]) of cache.pooled (see include/kpool.h)."""
    n = _compress_args("kpool_compress", dims, cache, keys, gates, ape, pool_seq, pool_id, src)
    _check("kpool_compress", load().kpool_compress(ctypes.byref(dims.c()), ctypes.byref(cache.c()), n,
                                                   _ptr(keys), _ptr(gates), _ptr(src), _ptr(ape), _ptr(pool_seq),
                                                   _ptr(pool_id), _stream(stream)))


def dsa_indexer_score(dims: Dims, cache: Cache, queries: Queries, q_idx, w, scores, stream=None) -> None:
    """scores[q, p] for p < (pos[q] + 1) / P; scores is fp32 [n_q, ld]."""
    _score_args("dsa_indexer_score", dims, cache, queries, q_idx, w, scores)
    _check("dsa_indexer_score", load().dsa_indexer_score(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                                         ctypes.byref(queries.c()), _ptr(q_idx), _ptr(w),
                                                         _ptr(scores), int(scores.stride(0)), _stream(stream)))


def dsa_compress_score(dims: Dims, cache: Cache, keys, gates, ape, pool_seq, pool_id, queries: Queries, q_idx, w,
                       scores, src=None, stream=None) -> None:
    """kpool_compress(...) then dsa_indexer_score(...) as one call: a decode batch with at most 64 pools to pool
    takes one launch (see include/kpool.h)."""
    fn = "dsa_compress_score"
    n = _compress_args(fn, dims, cache, keys, gates, ape, pool_seq, pool_id, src)
    _score_args(fn, dims, cache, queries, q_idx, w, scores)
    _check(fn, load().dsa_compress_score(ctypes.byref(dims.c()), ctypes.byref(cache.c()), n, _ptr(keys),
                                         _ptr(gates), _ptr(src), _ptr(ape), _ptr(pool_seq), _ptr(pool_id),
                                         ctypes.byref(queries.c()), _ptr(q_idx), _ptr(w), _ptr(scores),
                                         int(scores.stride(0)), _stream(stream)))


def dsa_topk_workspace_size(dims: Dims, queries: Queries) -> int:
    return int(load().dsa_topk_workspace_size(ctypes.byref(dims.c()), ctypes.byref(queries.c())))


def dsa_topk_select(dims: Dims, queries: Queries, scores, sel, n_sel, workspace=None, stream=None) -> None:
    """sel [n_q, k] int32 ascending pool ids padded with -1; n_sel [n_q] int32."""
    import torch
    fn = "dsa_topk_select"
    n = _check_queries(fn, queries)
    _want(fn, "scores", scores, (torch.float32,), (n, None), rows_only=True, min_rows=True)
    _want(fn, "sel", sel, _i32(), (n, dims.topk), min_rows=True)
    _want(fn, "n_sel", n_sel, _i32(), (n,), min_rows=True)
    if workspace is not None:
        _want(fn, "workspace", workspace, (workspace.dtype,), tuple(workspace.shape))
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("dsa_topk_select", load().dsa_topk_select(ctypes.byref(dims.c()), ctypes.byref(queries.c()),
                                                     _ptr(scores), int(scores.stride(0)), _ptr(sel), _ptr(n_sel),
                                                     _ptr(workspace), ws_bytes, _stream(stream)))


def sparse_mla_workspace_size(dims: Dims, queries: Queries) -> int:
    return int(load().sparse_mla_workspace_size(ctypes.byref(dims.c()), ctypes.byref(queries.c())))


def _check_attn(fn: str, dims: Dims, cache: Cache, queries: Queries, q, sel, n_sel, out, lse, workspace,
                fp8: bool = False, sel_row=None, runs: bool = False) -> None:
    import torch
    n = _check_queries(fn, queries)
    st = _storage(dims)
    _want(fn, "cache.latent", cache.latent, (torch.uint8,) if fp8 else st, (None, dims.page_tokens, dims.latent_dim))
    _want(fn, "q", q, st, (n, dims.heads, dims.latent_dim), min_rows=True)
    rows = (n + 1) // 2 if runs else n if sel_row is None else None
    _want(fn, "sel", sel, _i32(), (rows, dims.topk), min_rows=True)
    _want(fn, "n_sel", n_sel, _i32(), (sel.shape[0],), min_rows=True)
    if sel_row is not None:
        _want(fn, "sel_row", sel_row, _i32(), (n,))
    _want(fn, "out", out, st, (n, dims.heads, dims.v_dim), min_rows=True)
    if lse is not None:
        _want(fn, "lse", lse, (torch.float32,), (n, dims.heads), min_rows=True)
    if workspace is not None:
        _want(fn, "workspace", workspace, (workspace.dtype,), tuple(workspace.shape))


def sparse_mla_attn(dims: Dims, cache: Cache, queries: Queries, q, sel, n_sel, out, lse=None, workspace=None,
                    stream=None) -> None:
    """out [n_q, H, V] (storage dtype), lse [n_q, H] fp32 (optional)."""
    _check_attn("sparse_mla_attn", dims, cache, queries, q, sel, n_sel, out, lse, workspace)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("sparse_mla_attn", load().sparse_mla_attn(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                                     ctypes.byref(queries.c()), _ptr(q), _ptr(sel), _ptr(n_sel),
                                                     _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                                     _stream(stream)))


def sparse_mla_attn_shared(dims: Dims, cache: Cache, queries: Queries, q, sel, n_sel, sel_row, out, lse=None,
                           workspace=None, stream=None) -> None:
    """As sparse_mla_attn, query i attending selection row sel_row[i] (int32 [n_q]) cut at its own position, plus its
    own incomplete trailing pool (see include/kpool.h)."""
    _check_attn("sparse_mla_attn_shared", dims, cache, queries, q, sel, n_sel, out, lse, workspace, sel_row=sel_row)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("sparse_mla_attn_shared", load().sparse_mla_attn_shared(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                                                   ctypes.byref(queries.c()), _ptr(q), _ptr(sel),
                                                                   _ptr(n_sel), _ptr(sel_row), _ptr(out), _ptr(lse),
                                                                   _ptr(workspace), ws_bytes, _stream(stream)))


def sparse_mla_mtp_workspace_size(dims: Dims, queries: Queries) -> int:
    return int(load().sparse_mla_mtp_workspace_size(ctypes.byref(dims.c()), ctypes.byref(queries.c())))


def sparse_mla_attn_mtp(dims: Dims, cache: Cache, queries: Queries, q, sel, n_sel, out, lse=None, workspace=None,
                        stream=None) -> None:
    """MTP verification: queries 2r (target) and 2r + 1 (draft) attend selection row r (sel has ceil(n_q / 2) rows),
    each as sparse_mla_attn_shared would with sel_row[i] = i // 2; one gather per run (see include/kpool.h)."""
    _check_attn("sparse_mla_attn_mtp", dims, cache, queries, q, sel, n_sel, out, lse, workspace, runs=True)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("sparse_mla_attn_mtp", load().sparse_mla_attn_mtp(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                                             ctypes.byref(queries.c()), _ptr(q), _ptr(sel),
                                                             _ptr(n_sel), _ptr(out), _ptr(lse), _ptr(workspace),
                                                             ws_bytes, _stream(stream)))


def read_rows(base, row_bytes: int, rows, blocks_per_cu: int = 2, stream=None) -> None:
    """kp_read_rows: read the rows `rows` (int32 device tensor) of `base` (a device tensor whose first dimension
    indexes rows; row stride = its stride(0) in bytes) and discard them -- the gather-bandwidth reference."""
    fn = "kp_read_rows"
    _want(fn, "rows", rows, _i32(), (rows.numel(),))
    stride = base.stride(0) * base.element_size()
    _check(fn, load().kp_read_rows(_ptr(base), stride, int(row_bytes), _ptr(rows), int(rows.numel()),
                                   int(blocks_per_cu), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 36 << 20    # KP_NOALLOC_SCRATCH_BYTES of include/kpool.h


def sparse_mla_attn_noalloc(dims: Dims, cache: Cache, queries: Queries, q, sel, n_sel, out, lse=None,
                            stream=None) -> None:
    """As sparse_mla_attn with no workspace: the split-KV partials use the library's static per-device scratch of
    NOALLOC_SCRATCH_BYTES (calls that overlap on one GPU race; see include/kpool.h)."""
    _check_attn("sparse_mla_attn_noalloc", dims, cache, queries, q, sel, n_sel, out, lse, None)
    _check("sparse_mla_attn_noalloc", load().sparse_mla_attn_noalloc(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                                                     ctypes.byref(queries.c()), _ptr(q), _ptr(sel),
                                                                     _ptr(n_sel), _ptr(out), _ptr(lse),
                                                                     _stream(stream)))


def sparse_mla_attn_fp8(dims: Dims, cache: Cache, queries: Queries, q, sel, n_sel, kv_scale: float, out, lse=None,
                        workspace=None, stream=None) -> None:
    """As sparse_mla_attn, over a latent cache of E4M3 codes (cache.latent uint8) scaled by kv_scale."""
    _check_attn("sparse_mla_attn_fp8", dims, cache, queries, q, sel, n_sel, out, lse, workspace, fp8=True)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("sparse_mla_attn_fp8", load().sparse_mla_attn_fp8(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                                             ctypes.byref(queries.c()), _ptr(q), _ptr(sel),
                                                             _ptr(n_sel), float(kv_scale), _ptr(out), _ptr(lse),
                                                             _ptr(workspace), ws_bytes, _stream(stream)))


# ----------------------------------------------------------------------------------------------------------
# the dense projections beside the path (kp_linear)
# ----------------------------------------------------------------------------------------------------------
def _mat3(t, name: str):
    """(batch, rows, ld, batch stride) of a 2-D [rows, cols] or 3-D [batch, rows, cols] view, cols contiguous."""
    if t.dim() == 2:
        b, rows, ld, sb = 1, t.shape[0], t.stride(0), 0
    elif t.dim() == 3:
        b, rows, ld, sb = t.shape[0], t.shape[1], t.stride(1), t.stride(0)
    else:
        raise ValueError(f"kp_linear: {name} must be 2-D or 3-D")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"kp_linear: {name} needs a contiguous last dimension")
    return b, rows, ld, sb


def linear_workspace_size(batch: int, M: int, N: int, K: int) -> int:
    """Bytes of split-K workspace kp_linear can use for this shape (0: it never splits)."""
    return int(load().kp_linear_workspace_size(batch, M, N, K))


def _problem(a, w, out, alpha: float = 1.0) -> _LinearProblem:
    """The kp_linear_problem of out[b] = alpha * a[b] @ w[b]^T (see linear)."""
    import torch
    ba, M, lda, sa = _mat3(a, "a")
    bw, N, ldw, sw = _mat3(w, "w")
    bc, Mc, ldc, sc = _mat3(out, "out")
    batch = max(ba, bw, bc)
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("kp_linear: a and w must be bfloat16")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("kp_linear: out must be bfloat16 or float32")
    if any(x not in (1, batch) for x in (ba, bw, bc)) or bc != batch or Mc != M or out.shape[-1] != N \
            or w.shape[-1] != a.shape[-1]:
        raise ValueError(f"kp_linear: shapes {tuple(a.shape)} x {tuple(w.shape)} -> {tuple(out.shape)} disagree")
    c_dtype = KP_DTYPE_BF16 if out.dtype == torch.bfloat16 else KP_DTYPE_F32
    return _LinearProblem(batch, M, N, a.shape[-1], _ptr(a), lda, sa, _ptr(w), ldw, sw, _ptr(out), ldc, sc, c_dtype,
                          float(alpha))


def linear(a, w, out, alpha: float = 1.0, workspace=None, stream=None) -> None:
    """out[b] = alpha * a[b] @ w[b]^T (kp_linear).  a [.., M, K] and w [.., N, K] bf16; out [.., M, N] bf16 or
    float32.  2-D operands are shared by every batch entry; 3-D ones give the batch (views with any row and batch
    strides, last dimension contiguous).  workspace: a device tensor of at least linear_workspace_size(...) bytes
    (any contents), reused across calls (None: no split-K)."""
    q = _problem(a, w, out, alpha)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("kp_linear", load().kp_linear(q.batch, q.M, q.N, q.K, q.A, q.lda, q.stride_a, q.W, q.ldw, q.stride_w, q.C,
                                         q.ldc, q.stride_c, q.c_dtype, q.alpha, _ptr(workspace), ws_bytes,
                                         _stream(stream)))


def _problems(products):
    arr = (_LinearProblem * max(len(products), 1))()
    for i, p in enumerate(products):
        arr[i] = _problem(*p)
    return arr


def linear_shapes_workspace_size(shapes) -> int:
    """Split-K workspace of a group given only its shapes [(batch, M, N, K, c_dtype), ...] (nothing is read)."""
    arr = (_LinearProblem * max(len(shapes), 1))()
    for i, (b, M, N, K, dt) in enumerate(shapes):
        # stand-in operands: aligned, never dereferenced by the size query
        arr[i] = _LinearProblem(b, M, N, K, 256, K, 0, 256, K, 0, 256, (N + 3) // 4 * 4, 0, dt, 1.0)
    return int(load().kp_linear_group_workspace_size(len(shapes), arr))


def linear_group_workspace_size(products) -> int:
    """Bytes of split-K workspace for a group of products [(a, w, out[, alpha]), ...]."""
    return int(load().kp_linear_group_workspace_size(len(products), _problems(products)))


def linear_group(products, workspace=None, stream=None) -> None:
    """Up to 8 independent products [(a, w, out[, alpha]), ...] in one launch (kp_linear_group)."""
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check("kp_linear_group", load().kp_linear_group(len(products), _problems(products), _ptr(workspace), ws_bytes,
                                                     _stream(stream)))


def indexer_products(x, cq, w_q, w_w, w_kg, q_idx, w, keys, gates):
    """The indexer's four products for linear_group: q_idx [T, Hi, D] = cq @ w_q^T (head-major), w [T, Hi] (float32)
    = x @ w_w^T, keys | gates [T, D] = x @ w_kg^T split after D columns (key first)."""
    T, D = x.shape[0], keys.shape[-1]
    return [(cq, w_q, q_idx.view(T, -1)), (x, w_w, w), (x, w_kg[:D], keys), (x, w_kg[D:2 * D], gates)]


def absorb_product(q_nope, w_uk_t, q):
    """The query absorb as a product for linear_group (see mla_absorb_q)."""
    V = w_uk_t.shape[1]
    return (q_nope.transpose(0, 1), w_uk_t, q[:, :, :V].transpose(0, 1))


def indexer_project(x, cq, w_q, w_w, w_kg, q_idx, w, keys, gates, workspace=None, stream=None) -> None:
    """The indexer's projections in one grouped launch (see indexer_products)."""
    linear_group(indexer_products(x, cq, w_q, w_w, w_kg, q_idx, w, keys, gates), workspace=workspace, stream=stream)


def mla_absorb_q(q_nope, w_uk_t, q, workspace=None, stream=None) -> None:
    """Query in latent space, per head: q[t, h, :V] = W_UK[h]^T q_nope[t, h].  q_nope [T, H, dn] bf16, w_uk_t
    [H, V, dn] (W_UK[h] transposed, prepared once), q [T, H, L] bf16 (columns V..L-1 are left as they are)."""
    linear(*absorb_product(q_nope, w_uk_t, q), workspace=workspace, stream=stream)


def mla_unabsorb_o(o_lat, w_uv, o, workspace=None, stream=None) -> None:
    """Head output from the latent output: o[t, h] = W_UV[h] o_lat[t, h].  o_lat [T, H, V] bf16, w_uv [H, dv, V],
    o [T, H, dv] (bf16 or float32)."""
    linear(o_lat.transpose(0, 1), w_uv, o.transpose(0, 1), workspace=workspace, stream=stream)
