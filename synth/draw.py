"""Seeded draws and storage encodings.

Every tensor gets its own PCG64 stream, seeded from (workload seed, tensor
id, chunk id), so each tensor is reproducible on its own and large tensors
are drawn in parallel chunks without depending on the thread count.

Distributions: activations are N(0, 1) / sqrt(last dim) in float32, then
stored as float32, bfloat16 (round-to-nearest-even, torch's cast) or OCP
e4m3fn (per 128-row block: scale = block amax / 448, codes = torch's
float8_e4m3fn cast of value / scale).  Indexer head weights are
N(0, 1) / sqrt(h_idx) float32.  Decode context lengths are uniform integers
in [len_lo, len_hi]; physical pages are a seeded permutation of the pool.
"""

from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

from .workloads import Workload

_CHUNK = 1 << 22
_IDS = {"q_idx": 1, "w": 2, "k_idx": 3, "q": 4, "kv": 5, "input_ids": 6,
        "lengths": 7, "pages": 8, "own_pages": 9}
FP8_BLOCK_ROWS = 128
E4M3_MAX = 448.0


def _stream(seed: int, tensor: str, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), _IDS[tensor], int(chunk)])
    return np.random.Generator(np.random.PCG64(ss))


def _normal(seed: int, tensor: str, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, min(n, c + _CHUNK)) for c in range(0, n, _CHUNK)]

    def fill(i_lo_hi):
        i, (lo, hi) = i_lo_hi
        _stream(seed, tensor, i).standard_normal(hi - lo, dtype=np.float32,
                                                 out=out[lo:hi])
        out[lo:hi] *= np.float32(std)

    workers = min(len(chunks), max(1, min(16, os.cpu_count() or 1)))
    if workers > 1:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, enumerate(chunks)))
    else:
        for item in enumerate(chunks):
            fill(item)
    return out.reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_blocks(x: np.ndarray):
    """Per-128-row block scaled e4m3fn codes of a [rows, cols] array."""
    rows = x.shape[0]
    nblk = -(-rows // FP8_BLOCK_ROWS)
    pad = nblk * FP8_BLOCK_ROWS - rows
    xb = np.concatenate([x, np.zeros((pad,) + x.shape[1:], np.float32)]) \
        if pad else x
    xb = xb.reshape(nblk, FP8_BLOCK_ROWS, -1)
    amax = np.abs(xb).max(axis=(1, 2))
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), 1.0).astype(np.float32)
    scaled = np.clip(xb / scale[:, None, None], -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(scaled, dtype=np.float32)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes = codes.reshape(nblk * FP8_BLOCK_ROWS, *x.shape[1:])[:rows]
    return np.ascontiguousarray(codes), scale


def _store(x: np.ndarray, fmt: str):
    if fmt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32), None
    if fmt == "bf16":
        return to_bf16_bits(x), None
    if fmt == "fp8":
        return to_e4m3fn_blocks(x)
    raise ValueError(fmt)


def draw_prefill(wl: Workload, n_local: int) -> dict:
    """Inputs of one rank's prefill step.

    ``n_local`` is the number of queries the rank owns (the caller supplies
    it).  Token-indexed tensors (``k_idx``, ``kv``, ``input_ids``) cover all
    ``T`` tokens in logical order -- what the ranks' own projections produce
    together; query tensors cover the rank's ``n_local`` queries.
    """
    assert wl.kind == "prefill"
    T = wl.num_tokens
    s = wl.seed
    out = {"cu_seqlens": np.asarray(wl.cu_seqlens(), dtype=np.int32)}
    out["input_ids"] = _stream(s, "input_ids").integers(
        0, 1 << 17, size=T, dtype=np.int32)
    q_idx = _normal(s, "q_idx", (n_local, wl.h_idx, wl.d_idx), wl.d_idx ** -0.5)
    out["q_idx"], _ = _store(q_idx, wl.act_fmt)
    out["w"] = _normal(s, "w", (n_local, wl.h_idx), wl.h_idx ** -0.5)
    k_idx = _normal(s, "k_idx", (T, wl.d_idx), wl.d_idx ** -0.5)
    out["k_idx"], out["k_idx_scale"] = _store(k_idx, wl.kv_fmt)
    q = _normal(s, "q", (n_local, wl.n_heads, wl.d_qk), wl.d_qk ** -0.5)
    out["q"], _ = _store(q, wl.act_fmt)
    kv = _normal(s, "kv", (T, wl.d_qk), wl.d_qk ** -0.5)
    out["kv"], out["kv_scale"] = _store(kv, wl.kv_fmt)
    return out


def draw_page_table(counts, page_size: int, seed: int, spare: int = 0):
    """A paged pool holding ``counts[b]`` rows for request ``b``: every
    request gets ceil(counts[b] / page_size) pages of a seeded random
    permutation of the pool's pages (plus ``spare`` unused ones).  Returns
    (page_table [n_req, max_pages] int32 with -1 past a request's pages,
    pool_rows)."""
    pages = [-(-int(c) // page_size) for c in counts]
    n_pages = int(sum(pages)) + spare
    perm = _stream(seed, "own_pages").permutation(n_pages).astype(np.int32)
    table = np.full((len(pages), max(pages + [1])), -1, dtype=np.int32)
    off = 0
    for b, k in enumerate(pages):
        table[b, :k] = perm[off: off + k]
        off += k
    return table, n_pages * page_size


def draw_decode(wl: Workload) -> dict:
    """Inputs of one decode step: one query per request, paged KV pools."""
    assert wl.kind == "decode"
    s = wl.seed
    R = wl.n_req
    lengths = _stream(s, "lengths").integers(wl.len_lo, wl.len_hi + 1, size=R,
                                             dtype=np.int64)
    pages_per_req = [-(-int(L) // wl.page_size) for L in lengths]
    n_pages = int(sum(pages_per_req))
    perm = _stream(s, "pages").permutation(n_pages).astype(np.int32)
    max_pages = max(pages_per_req)
    table = np.full((R, max_pages), -1, dtype=np.int32)
    off = 0
    for i, npg in enumerate(pages_per_req):
        table[i, :npg] = perm[off: off + npg]
        off += npg
    pool_rows = n_pages * wl.page_size
    out = {"lengths": lengths.astype(np.int32), "page_table": table,
           "pool_rows": pool_rows}
    q_idx = _normal(s, "q_idx", (R, wl.h_idx, wl.d_idx), wl.d_idx ** -0.5)
    out["q_idx"], _ = _store(q_idx, wl.act_fmt)
    out["w"] = _normal(s, "w", (R, wl.h_idx), wl.h_idx ** -0.5)
    k_idx = _normal(s, "k_idx", (pool_rows, wl.d_idx), wl.d_idx ** -0.5)
    out["k_idx"], out["k_idx_scale"] = _store(k_idx, wl.kv_fmt)
    q = _normal(s, "q", (R, wl.n_heads, wl.d_qk), wl.d_qk ** -0.5)
    out["q"], _ = _store(q, wl.act_fmt)
    kv = _normal(s, "kv", (pool_rows, wl.d_qk), wl.d_qk ** -0.5)
    out["kv"], out["kv_scale"] = _store(kv, wl.kv_fmt)
    return out
