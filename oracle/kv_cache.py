"""Own-KV retention in the paged cache pool -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain enumeration
over the rank's own tokens.

Source: "[DeepSeek v3.2] 上下文并行详解", section 4 part 3, step D: once the
attention of a layer is done the gathered global KV is dropped, and each
rank keeps only the KV of the tokens it owns (rank 1 keeps K1, K5 of the
8-token example) in the device cache pool, for the decode steps that follow.

Readings taken where the page is silent (listed again in the design doc):

* the rank's cache for a request holds that request's own tokens in their
  local order (the order the split leaves them in), so own token ``p`` of
  request ``b`` is logical cache position ``p``;
* the pool is paged as in decode: logical position ``p`` of request ``b``
  is physical row ``page_table[b, p // page_size] * page_size +
  p % page_size``;
* a row whose request or page is not mapped (request outside the table, a
  page index past the table's width, a page id of -1, a physical row past
  the pool) is not stored; nothing else in the pool changes;
* rows are stored as given (the storage format of the pool is the one of
  the rows; no re-encoding) by :func:`own_kv_cache_write`;
* :func:`own_kv_cache_write_fp8` instead encodes each kept row as OCP
  e4m3fn codes with one fp32 scale per row (round-robin lifts the old
  split's "no FP8 KV cache" limit, section 1 of the same page).  The pages
  give no encoding; the reading taken: scale = row amax / 448 (448 is the
  largest e4m3fn value), code = the e4m3fn value nearest to x / scale,
  ties to the even code, with x / scale clamped to [-448, 448]; an all-zero
  row gets scale 0 and zero codes.  A scale per row (not per block of rows)
  keeps the rows of different requests, written at different times, apart:
  writing a row never re-encodes another.  The code decision is taken on
  float32 values (amax, the scale and x / scale, each rounded to float32),
  the precision the device computes them in.
"""

from __future__ import annotations

import numpy as np

from .sparse_attention import bf16_bits_to_f64, e4m3fn_to_f64

E4M3_MAX = 448.0


def own_cache_position(j: int, batch_idx, local_cu) -> tuple[int, int]:
    """Request and logical cache position of the rank's local token ``j``:
    its request ``batch_idx[j]`` and its index among that request's own
    tokens, ``j - local_cu[batch_idx[j]]``."""
    b = int(batch_idx[j])
    return b, j - int(local_cu[b])


def own_kv_cache_write(rows: np.ndarray, batch_idx, local_cu, page_table: np.ndarray,
                       page_size: int, pool: np.ndarray) -> np.ndarray:
    """Return a copy of ``pool`` with every local row ``rows[j]`` stored at
    the physical row of its request's cache position (rows that map to no
    stored row are dropped).  ``rows`` [n_local, ...], ``pool`` [pool_rows,
    ...] of the same dtype and row shape; ``page_table`` [n_req, max_pages].
    """
    out = np.array(pool, copy=True)
    n_req, max_pages = page_table.shape
    for j in range(len(rows)):
        b = int(batch_idx[j])
        if b < 0 or b >= n_req:
            continue
        _, p = own_cache_position(j, batch_idx, local_cu)
        pg = p // page_size
        if p < 0 or pg >= max_pages:
            continue
        page = int(page_table[b, pg])
        if page < 0:
            continue
        phys = page * page_size + p % page_size
        if phys >= len(out):
            continue
        out[phys] = rows[j]
    return out


def encode_e4m3fn(x) -> np.ndarray:
    """float values -> OCP e4m3fn codes (uint8), round to nearest, ties to
    the even code.  Defined by search: the sign bit is the input's sign bit,
    and the magnitude code is the one among the 127 finite non-negative
    codes (0x00 .. 0x7E, decoded by :func:`e4m3fn_to_f64`) whose value is
    nearest to |x|; of two equally near codes the even one (mantissa LSB 0)
    wins.  Inputs must lie in [-448, 448].  Parity: pinned against torch's
    float8_e4m3fn cast on representable values, midpoints and random
    values (tests/test_oracle_kv_cache.py)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3fn encoding needs finite values in [-448, 448]")
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = e4m3fn_to_f64(codes)                       # increasing in the code
    mag = np.abs(x).reshape(-1)
    hi = np.searchsorted(vals, mag, side="left")      # first value >= |x|
    hi = np.minimum(hi, codes.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - vals[lo], vals[hi] - mag
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = (d_hi == d_lo) & (hi != lo)
    pick = np.where(tie, np.where(hi % 2 == 0, hi, lo), pick)
    pick = np.where(vals[hi] == mag, hi, pick)        # exact values
    sign = (np.signbit(x.reshape(-1))).astype(np.uint8) << 7
    return (codes[pick] | sign).reshape(x.shape)


def encode_row_fp8(row_bf16) -> tuple[np.ndarray, np.float32]:
    """One row of bfloat16 bit patterns -> (e4m3fn codes, fp32 scale), per
    the reading in the module docstring (every step in float32)."""
    x = bf16_bits_to_f64(row_bf16).astype(np.float32)        # exact
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(E4M3_MAX))
    if scale == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0)
    q = (x / scale).astype(np.float32)                        # float32 division
    q = np.clip(q, -E4M3_MAX, E4M3_MAX)
    return encode_e4m3fn(q), scale


def own_kv_cache_write_fp8(rows_bf16: np.ndarray, batch_idx, local_cu, page_table: np.ndarray,
                           page_size: int, pool_codes: np.ndarray, pool_scale: np.ndarray):
    """The rank's own rows (bfloat16 bit patterns, [n_local, D]) encoded as
    e4m3fn with a scale per row and stored where :func:`own_kv_cache_write`
    stores the row; returns copies of (pool_codes [pool_rows, D] uint8,
    pool_scale [pool_rows] float32).  Rows that map nowhere are dropped."""
    codes = np.array(pool_codes, copy=True)
    scales = np.array(pool_scale, dtype=np.float32, copy=True)
    n_req, max_pages = page_table.shape
    for j in range(len(rows_bf16)):
        b, p = own_cache_position(j, batch_idx, local_cu)
        if b < 0 or b >= n_req or p < 0 or p // page_size >= max_pages:
            continue
        page = int(page_table[b, p // page_size])
        if page < 0:
            continue
        phys = page * page_size + p % page_size
        if phys >= len(codes):
            continue
        codes[phys], scales[phys] = encode_row_fp8(rows_bf16[j])
    return codes, scales
