"""ctypes binding of libds32cp.so (the C ABI in include/ds32cp.h).

Argument marshalling only: tensors are passed as device pointers with their
sizes, the stream is torch's current HIP stream, and every compute step
runs in the HIP library.  Output buffers may be passed in (nothing is
allocated then) or are allocated here with torch as plain device memory.
There is no fallback: if the library is missing, importing this module
raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DS32CP_LIB", os.path.join(_HERE, "libds32cp.so"))

DS_F32, DS_BF16, DS_FP8_E4M3FN, DS_FP8_E4M3FN_ROWSCALE = 0, 1, 2, 3
STATUS = {0: "DS_OK", 1: "DS_ERR_INVALID_ARG", 2: "DS_ERR_UNSUPPORTED",
          3: "DS_ERR_WORKSPACE", 4: "DS_ERR_HIP"}


class DS32CPError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"ds32cp HIP library not found at {LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'`")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_p, _i32, _i64, _sz, _f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_size_t, ctypes.c_float)
_SIGS = {
    "ds_abi_version": ([], _i32),
    "ds_last_error": ([], ctypes.c_char_p),
    "ds_cp_local_count": ([_i64, _i32, _i32], _i32),
    "cp_split_metadata": ([_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p,
                           _i64, _p], _i32),
    "decode_metadata": ([_p, _i32, _p, _p, _p, _p], _i32),
    "ds_cp_in_seq_local_count": ([_p, _i32, _i32, _i32], _i32),
    "cp_split_metadata_in_seq": ([_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p,
                                  _p, _i64, _p], _i32),
    "kv_rerange": ([_p, _i32, _i32, _i32, _i64, _p, _p], _i32),
    "kv_cache_write": ([_p, _i32, _i64, _p, _p, _i32, _p, _i32, _i32, _p, _i64, _p], _i32),
    "kv_cache_write_fp8": ([_p, _i32, _i32, _i32, _p, _p, _i32, _p, _i32, _i32, _p, _p, _i64,
                            _p], _i32),
    "indexer_topk_workspace_size": ([_i32, _i32], _sz),
    "indexer_topk": ([_p, _i32, _p, _p, _i32, _p, _i64, _p, _p, _p, _p, _i32, _i32,
                      _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _sz, _p], _i32),
    "indexer_scores": ([_p, _i32, _p, _p, _i32, _p, _i64, _p, _p, _p, _p, _i32, _i32,
                        _i32, _i32, _i32, _i32, _i32, _p, _i64, _p], _i32),
    "topk_select": ([_p, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _i64, _i32, _i32,
                     _i32, _p, _p, _p], _i32),
    "sparse_mla_prefill": ([_p, _i32, _p, _i32, _p, _i64, _p, _i32, _i32, _i32, _i32,
                            _i32, _f32, _p, _i32, _p, _p, _sz, _p], _i32),
    "sparse_mla_prefill_workspace_size": ([_i64, _i32], _sz),
    "sparse_mla_workspace_size": ([_i32, _i32, _i32, _i32], _sz),
    "sparse_mla_decode": ([_p, _i32, _p, _i32, _p, _i64, _p, _i32, _i32, _i32, _i32,
                           _i32, _f32, _p, _i32, _p, _p, _sz, _p], _i32),
    "gemm_bf16_nt_workspace_size": ([_i32, _i32, _i32, _i32], _sz),
    "gemm_bf16_nt": ([_p, _i64, _i64, _p, _i64, _i64, _p, _i32, _i64, _i64, _i32, _i32, _i32,
                      _i32, _p, _sz, _p], _i32),
    "sparse_mla_decode_noalloc_scratch_bytes": ([], _sz),
    "sparse_mla_decode_noalloc": ([_p, _i32, _p, _i32, _p, _i64, _p, _i32, _i32, _i32, _i32,
                                   _i32, _f32, _p, _i32, _p, _p], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DS32CPError(fn, status, lib.ds_last_error().decode(errors="replace"))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch tensor, got {type(t).__name__}")
    if t.numel() and not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2}


def dtype_code(t: torch.Tensor, scale_per_row: bool = False) -> int:
    """Storage code of a tensor; fp8 tensors carry one scale per 128 rows,
    or one per row with scale_per_row (the pools kv_cache_write_fp8 fills)."""
    if t.dtype == torch.float32:
        return DS_F32
    if t.dtype == torch.bfloat16:
        return DS_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DS_FP8_E4M3FN_ROWSCALE if scale_per_row else DS_FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


def _i32buf(n, device, out):
    if out is not None:
        return out
    return torch.empty(max(n, 0), dtype=torch.int32, device=device)


# --------------------------------------------------------------------- api

def abi_version() -> int:
    return lib.ds_abi_version()


def cp_local_count(num_tokens: int, cp_size: int, cp_rank: int) -> int:
    n = lib.ds_cp_local_count(num_tokens, cp_size, cp_rank)
    if n < 0:
        raise ValueError("invalid cp_size / cp_rank / num_tokens")
    return n


def cp_split_metadata(cu_seqlens: torch.Tensor, num_tokens: int, cp_size: int,
                      cp_rank: int, rows_src: torch.Tensor | None = None,
                      out: dict | None = None, stream=None) -> dict:
    """Step 1.  Returns dict with local_cu, batch_idx, global_idx, kv_start,
    kv_len (and rows when rows_src is given)."""
    dev = cu_seqlens.device
    B = cu_seqlens.numel() - 1
    n = cp_local_count(num_tokens, cp_size, cp_rank)
    out = dict(out or {})
    res = {
        "local_cu": _i32buf(B + 1, dev, out.get("local_cu")),
        "batch_idx": _i32buf(n, dev, out.get("batch_idx")),
        "global_idx": _i32buf(n, dev, out.get("global_idx")),
        "kv_start": _i32buf(n, dev, out.get("kv_start")),
        "kv_len": _i32buf(n, dev, out.get("kv_len")),
    }
    row_bytes = 0
    if rows_src is not None:
        row_bytes = rows_src.element_size() * math.prod(rows_src.shape[1:])
        rows = out.get("rows")
        if rows is None:
            rows = torch.empty((n,) + tuple(rows_src.shape[1:]), dtype=rows_src.dtype, device=dev)
        res["rows"] = rows
    st = lib.cp_split_metadata(
        _ptr(cu_seqlens), B, num_tokens, cp_size, cp_rank, _ptr(res["local_cu"]),
        _ptr(res["batch_idx"]), _ptr(res["global_idx"]), _ptr(res["kv_start"]),
        _ptr(res["kv_len"]), _ptr(rows_src), _ptr(res.get("rows")), row_bytes,
        _stream(stream))
    _check("cp_split_metadata", st)
    return res


def cp_in_seq_local_count(cu_seqlens_host, cp_size: int, cp_rank: int) -> int:
    """Tokens of rank cp_rank under the in-sequence split (host offsets)."""
    cu = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    n = lib.ds_cp_in_seq_local_count(ctypes.cast(cu, ctypes.c_void_p), len(cu_seqlens_host) - 1,
                                     cp_size, cp_rank)
    if n < 0:
        raise ValueError("invalid cu_seqlens / cp_size / cp_rank")
    return n


def cp_split_metadata_in_seq(cu_seqlens: torch.Tensor, num_tokens: int, cp_size: int,
                             cp_rank: int, n_local: int | None = None,
                             rows_src: torch.Tensor | None = None, out: dict | None = None,
                             stream=None) -> dict:
    """Contrast mode (in-sequence split).  Same fields as cp_split_metadata;
    n_local defaults to the count from a host copy of cu_seqlens."""
    dev = cu_seqlens.device
    B = cu_seqlens.numel() - 1
    if n_local is None:
        n_local = cp_in_seq_local_count(cu_seqlens.cpu().tolist(), cp_size, cp_rank)
    out = dict(out or {})
    res = {
        "local_cu": _i32buf(B + 1, dev, out.get("local_cu")),
        "batch_idx": _i32buf(n_local, dev, out.get("batch_idx")),
        "global_idx": _i32buf(n_local, dev, out.get("global_idx")),
        "kv_start": _i32buf(n_local, dev, out.get("kv_start")),
        "kv_len": _i32buf(n_local, dev, out.get("kv_len")),
    }
    row_bytes = 0
    if rows_src is not None:
        row_bytes = rows_src.element_size() * math.prod(rows_src.shape[1:])
        rows = out.get("rows")
        if rows is None:
            rows = torch.empty((n_local,) + tuple(rows_src.shape[1:]), dtype=rows_src.dtype,
                               device=dev)
        res["rows"] = rows
    st = lib.cp_split_metadata_in_seq(
        _ptr(cu_seqlens), B, num_tokens, cp_size, cp_rank, n_local, _ptr(res["local_cu"]),
        _ptr(res["batch_idx"]), _ptr(res["global_idx"]), _ptr(res["kv_start"]),
        _ptr(res["kv_len"]), _ptr(rows_src), _ptr(res.get("rows")), row_bytes, _stream(stream))
    _check("cp_split_metadata_in_seq", st)
    return res


def kv_rerange(src: torch.Tensor, slot_rows: int, num_tokens: int, cp_size: int,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Step 2: rank-concatenated rows -> logical order (row = first axis)."""
    row_bytes = src.element_size() * math.prod(src.shape[1:])
    if out is None:
        out = torch.empty((num_tokens,) + tuple(src.shape[1:]), dtype=src.dtype,
                          device=src.device)
    st = lib.kv_rerange(_ptr(src), slot_rows, num_tokens, cp_size, row_bytes, _ptr(out),
                        _stream(stream))
    _check("kv_rerange", st)
    return out


def kv_cache_write(rows: torch.Tensor, batch_idx: torch.Tensor, local_cu: torch.Tensor,
                   page_table: torch.Tensor, page_size: int, pool: torch.Tensor,
                   stream=None) -> torch.Tensor:
    """Step D: store the rank's own rows (row = first axis) in the paged
    pool, in place; returns pool."""
    if rows.dtype != pool.dtype or tuple(rows.shape[1:]) != tuple(pool.shape[1:]):
        raise ValueError("rows and pool must have the same dtype and row shape")
    for name, t in (("batch_idx", batch_idx), ("local_cu", local_cu), ("page_table", page_table)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    n_req = local_cu.numel() - 1
    if batch_idx.numel() < rows.shape[0] or n_req < 0 or page_table.dim() != 2 \
            or page_table.shape[0] < n_req:
        raise ValueError("batch_idx needs a request per row, local_cu n_req + 1 entries, "
                         "page_table [n_req, max_pages]")
    row_bytes = rows.element_size() * math.prod(rows.shape[1:])
    st = lib.kv_cache_write(_ptr(rows), rows.shape[0], row_bytes, _ptr(batch_idx),
                            _ptr(local_cu), n_req, _ptr(page_table), page_table.shape[1], page_size,
                            _ptr(pool), pool.shape[0], _stream(stream))
    _check("kv_cache_write", st)
    return pool


def kv_cache_write_fp8(rows: torch.Tensor, batch_idx: torch.Tensor, local_cu: torch.Tensor,
                       page_table: torch.Tensor, page_size: int, pool_codes: torch.Tensor,
                       pool_scale: torch.Tensor, stream=None):
    """Step D with fp8 encoding: the rank's own bf16 rows [n_local, D] are
    encoded per row into the pool (codes [pool_rows, D] float8_e4m3fn or
    uint8, scales [pool_rows] fp32), in place; returns (pool_codes,
    pool_scale).  The pool then reads back with scale_per_row=True."""
    if rows.dtype != torch.bfloat16 or rows.dim() != 2:
        raise ValueError("rows must be a 2-d bf16 tensor")
    if tuple(pool_codes.shape[1:]) != tuple(rows.shape[1:]) or pool_codes.element_size() != 1:
        raise ValueError("pool_codes must be [pool_rows, D] of one-byte codes")
    if pool_scale.dtype != torch.float32 or pool_scale.numel() < pool_codes.shape[0]:
        raise ValueError("pool_scale must be fp32 with a scale per pool row")
    for name, t in (("batch_idx", batch_idx), ("local_cu", local_cu), ("page_table", page_table)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    n_req = local_cu.numel() - 1
    st = lib.kv_cache_write_fp8(_ptr(rows), DS_BF16, rows.shape[0], rows.shape[1], _ptr(batch_idx),
                                _ptr(local_cu), n_req, _ptr(page_table), page_table.shape[1],
                                page_size, _ptr(pool_codes), _ptr(pool_scale),
                                pool_codes.shape[0], _stream(stream))
    _check("kv_cache_write_fp8", st)
    return pool_codes, pool_scale


def indexer_topk_workspace_size(n_q: int, max_kv_len: int) -> int:
    return lib.indexer_topk_workspace_size(n_q, max_kv_len)


def _paging(q_req, page_table, page_size):
    if page_table is None:
        return None, None, 0, 0, 0
    return (_ptr(q_req), _ptr(page_table), page_table.shape[0], page_size,
            page_table.shape[1])


def indexer_topk(q_idx, w, k_idx, kv_start, kv_len, max_kv_len: int, topk: int,
                 k_scale=None, q_req=None, page_table=None, page_size: int = 0,
                 topk_idx=None, topk_score=None, want_score: bool = False,
                 workspace=None, scale_per_row: bool = False, stream=None):
    """Steps 3 + 4.  Returns (topk_idx [n_q, topk] int32, topk_score or None)."""
    n_q, h_idx, d_idx = q_idx.shape
    dev = q_idx.device
    if topk_idx is None:
        topk_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if want_score and topk_score is None:
        topk_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    ws_bytes = indexer_topk_workspace_size(n_q, max_kv_len)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    qr, pt, n_req, ps, mp = _paging(q_req, page_table, page_size)
    st = lib.indexer_topk(
        _ptr(q_idx), dtype_code(q_idx), _ptr(w), _ptr(k_idx), dtype_code(k_idx, scale_per_row),
        _ptr(k_scale), k_idx.shape[0], _ptr(kv_start), _ptr(kv_len), qr, pt, n_req, ps, mp,
        n_q, h_idx, d_idx, max_kv_len, topk, _ptr(topk_idx), _ptr(topk_score),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("indexer_topk", st)
    return topk_idx, topk_score


def indexer_scores(q_idx, w, k_idx, kv_start, kv_len, max_kv_len: int, k_scale=None,
                   q_req=None, page_table=None, page_size: int = 0, scores=None,
                   scale_per_row: bool = False, stream=None) -> torch.Tensor:
    """Step 3 alone: scores [n_q, max_kv_len] fp32 (entries past kv_len are
    left as allocated: NaN when allocated here)."""
    n_q, h_idx, d_idx = q_idx.shape
    if scores is None:
        scores = torch.full((n_q, max(max_kv_len, 1)), float("nan"), dtype=torch.float32,
                            device=q_idx.device)
    qr, pt, n_req, ps, mp = _paging(q_req, page_table, page_size)
    st = lib.indexer_scores(
        _ptr(q_idx), dtype_code(q_idx), _ptr(w), _ptr(k_idx), dtype_code(k_idx, scale_per_row),
        _ptr(k_scale), k_idx.shape[0], _ptr(kv_start), _ptr(kv_len), qr, pt, n_req, ps, mp,
        n_q, h_idx, d_idx, max_kv_len, _ptr(scores), scores.shape[1], _stream(stream))
    _check("indexer_scores", st)
    return scores


def topk_select(scores, kv_start, kv_len, max_kv_len: int, topk: int, k_rows: int,
                q_req=None, page_table=None, page_size: int = 0, topk_idx=None,
                topk_score=None, want_score: bool = False, stream=None):
    n_q = scores.shape[0]
    dev = scores.device
    if topk_idx is None:
        topk_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if want_score and topk_score is None:
        topk_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    qr, pt, n_req, ps, mp = _paging(q_req, page_table, page_size)
    st = lib.topk_select(_ptr(scores), scores.shape[1], _ptr(kv_start), _ptr(kv_len), qr, pt,
                         n_req, ps, mp, k_rows, n_q, max_kv_len, topk, _ptr(topk_idx),
                         _ptr(topk_score), _stream(stream))
    _check("topk_select", st)
    return topk_idx, topk_score


def _mla_common(q, kv, topk_idx, d_latent, out, out_dtype):
    n_q, n_heads, d_qk = q.shape
    if out is None:
        out = torch.empty((n_q, n_heads, d_latent), dtype=out_dtype, device=q.device)
    return n_q, n_heads, d_qk - d_latent, out


def sparse_mla_prefill_workspace_size(kv_rows: int, kv_dtype) -> int:
    return lib.sparse_mla_prefill_workspace_size(kv_rows, _DTYPES[kv_dtype])


def sparse_mla_prefill(q, kv, topk_idx, sm_scale: float, d_latent: int, kv_scale=None,
                       out=None, out_dtype=None, lse=None, want_lse: bool = True,
                       workspace=None, scale_per_row: bool = False, stream=None):
    """Step 5 (prefill).  Returns (out [n_q, H, d_latent], lse [n_q, H] or None).
    fp8 kv needs a workspace (allocated here when not given)."""
    out_dtype = out_dtype or (torch.float32 if q.dtype == torch.float32 else torch.bfloat16)
    n_q, H, d_rope, out = _mla_common(q, kv, topk_idx, d_latent, out, out_dtype)
    if want_lse and lse is None:
        lse = torch.empty((n_q, H), dtype=torch.float32, device=q.device)
    need = sparse_mla_prefill_workspace_size(kv.shape[0], kv.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.sparse_mla_prefill(
        _ptr(q), dtype_code(q), _ptr(kv), dtype_code(kv, scale_per_row), _ptr(kv_scale), kv.shape[0],
        _ptr(topk_idx), n_q, H, d_latent, d_rope, topk_idx.shape[1], sm_scale, _ptr(out),
        dtype_code(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check("sparse_mla_prefill", st)
    return out, lse


def sparse_mla_workspace_size(n_q: int, n_heads: int, d_latent: int, topk: int) -> int:
    return lib.sparse_mla_workspace_size(n_q, n_heads, d_latent, topk)


def sparse_mla_decode(q, kv, topk_idx, sm_scale: float, d_latent: int, kv_scale=None,
                      out=None, out_dtype=None, lse=None, want_lse: bool = True,
                      workspace=None, scale_per_row: bool = False, stream=None):
    """Step 5 (decode: rows split across workgroups, merged by LSE)."""
    out_dtype = out_dtype or (torch.float32 if q.dtype == torch.float32 else torch.bfloat16)
    n_q, H, d_rope, out = _mla_common(q, kv, topk_idx, d_latent, out, out_dtype)
    if want_lse and lse is None:
        lse = torch.empty((n_q, H), dtype=torch.float32, device=q.device)
    topk = topk_idx.shape[1]
    ws_bytes = sparse_mla_workspace_size(n_q, H, d_latent, topk)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib.sparse_mla_decode(
        _ptr(q), dtype_code(q), _ptr(kv), dtype_code(kv, scale_per_row), _ptr(kv_scale), kv.shape[0],
        _ptr(topk_idx), n_q, H, d_latent, d_rope, topk, sm_scale, _ptr(out), dtype_code(out),
        _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("sparse_mla_decode", st)
    return out, lse


def sparse_mla_decode_noalloc(q, kv, topk_idx, sm_scale: float, d_latent: int, *, out,
                              lse=None, kv_scale=None, scale_per_row: bool = False, stream=None):
    """Step 5 (decode) with the library's own scratch for the split partials:
    nothing is allocated, by this call or the library; the caller passes
    every output buffer."""
    n_q, H, d_qk = q.shape
    st = lib.sparse_mla_decode_noalloc(
        _ptr(q), dtype_code(q), _ptr(kv), dtype_code(kv, scale_per_row), _ptr(kv_scale), kv.shape[0],
        _ptr(topk_idx), n_q, H, d_latent, d_qk - d_latent, topk_idx.shape[1], sm_scale, _ptr(out),
        dtype_code(out), _ptr(lse), _stream(stream))
    _check("sparse_mla_decode_noalloc", st)
    return out, lse


def _gemm_operand(t: torch.Tensor, name: str):
    """(pointer, rows, cols, leading dim, batch, batch stride) of a 2-d
    [rows, cols] or 3-d [batch, rows, cols] view whose last dim is dense."""
    if t.dim() == 2:
        t3 = t.unsqueeze(0)
    elif t.dim() == 3:
        t3 = t
    else:
        raise ValueError(f"{name} must be 2-d or 3-d")
    if t3.shape[2] > 1 and t3.stride(2) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    batch_stride = t3.stride(0) if t3.shape[0] > 1 else 0
    return t3.data_ptr(), t3.shape[1], t3.shape[2], t3.stride(1), t3.shape[0], batch_stride


def gemm_bf16_nt_workspace_size(M: int, N: int, K: int, batch: int = 1) -> int:
    return lib.gemm_bf16_nt_workspace_size(M, N, K, batch)


def gemm_bf16_nt(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                 out_dtype=torch.bfloat16, workspace=None, stream=None) -> torch.Tensor:
    """C = A . B^T per batch: a [.., M, K], b [.., N, K] (weights as
    [out, in]), out [.., M, N]; 2-d or 3-d views whose last dimension is
    dense (strided per-head slices are passed in place)."""
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("a and b must be bf16")
    pa, M, K, lda, ba, sa = _gemm_operand(a, "a")
    pb, N, Kb, ldb, bb, sb = _gemm_operand(b, "b")
    batch = max(ba, bb)
    if Kb != K or ba not in (1, batch) or bb not in (1, batch):
        raise ValueError("a [.., M, K] and b [.., N, K] must agree in K and batch")
    if out is None:
        shape = (batch, M, N) if a.dim() == 3 or b.dim() == 3 else (M, N)
        out = torch.empty(shape, dtype=out_dtype, device=a.device)
    pc, Mc, Nc, ldc, bc, scs = _gemm_operand(out, "out")
    if (Mc, Nc) != (M, N) or bc not in (1, batch):
        raise ValueError("out must be [.., M, N]")
    need = gemm_bf16_nt_workspace_size(M, N, K, batch)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    st = lib.gemm_bf16_nt(pa, lda, sa, pb, ldb, sb, pc, dtype_code(out), ldc, scs, M, N, K,
                          batch, _ptr(workspace) if need else None,
                          workspace.numel() if need else 0, _stream(stream))
    _check("gemm_bf16_nt", st)
    return out


def decode_metadata(lengths: torch.Tensor, out: dict | None = None, stream=None) -> dict:
    """Decode step metadata (q_req, kv_start, kv_len) from the per-request
    context lengths (int32 on the device)."""
    if lengths.dtype != torch.int32:
        raise TypeError("lengths must be int32")
    n = lengths.numel()
    dev = lengths.device
    out = dict(out or {})
    res = {k: _i32buf(n, dev, out.get(k)) for k in ("q_req", "kv_start", "kv_len")}
    st = lib.decode_metadata(_ptr(lengths), n, _ptr(res["q_req"]), _ptr(res["kv_start"]),
                             _ptr(res["kv_len"]), _stream(stream))
    _check("decode_metadata", st)
    return res
