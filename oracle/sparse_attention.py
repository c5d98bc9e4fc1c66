"""Indexer scores, top-k selection and sparse latent attention -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain NumPy in
float64, one query at a time, no blocking or fusion.

Sources:

* "[RFC]: Parallel strategy for Deepseek v3.2 like models", comment thread:
  the indexer is the per-query selection of the top-k history KV entries
  (one pass per query over its history), and sparse MLA lets each query
  attend only to those top-k entries instead of to every key.
* "[DeepSeek v3.2] 上下文并行详解", section 2C: the indexer's KV range and
  the top-k index transform are expressed against the logically ordered KV
  after the rerange; section 4 part 3, step C: the rank's local queries
  attend to the complete (all-gathered) KV; the causal example there (T5
  attends to T0..T4).
* "Model Parallel Strategy Analysis" (Ascend skill page), common-errors
  table and the scenario-adjustment note: MLA's compressed KV is one latent
  vector per token, not stored per head, so all heads read the same row.

The pages give no formula for the indexer or for MLA.  The readings used
here (each also listed in the design doc):

* indexer score of query ``j`` against key row ``s``:
  ``I[j, s] = sum_h w[j, h] * max(0, <qI[j, h, :], kI[s, :]>)`` -- one
  indexer key per token shared by all indexer heads, per-query per-head
  weights, no extra scale;
* top-k: the ``k`` largest scores of the query's causal keys, ties to the
  lower key position; fewer than ``k`` causal keys -> all of them, then -1;
* sparse MLA in absorbed (latent, MQA-style) form: key = the full latent row
  (``d_latent + d_rope`` values, rope part already rotated), value = its
  first ``d_latent`` values, every head shares the row; softmax over the
  selected keys of ``sm_scale * <q, key>`` with natural exp;
  ``lse = max + log(sum(exp(logit - max)))``;
* fp8 storage is OCP e4m3fn (bias 7, no infinities, S.1111.111 = NaN) with
  one fp32 scale per 128 consecutive rows: value = code * scale.
"""

from __future__ import annotations

import numpy as np

FP8_BLOCK_ROWS = 128


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    bfloat16 is the upper half of an IEEE-754 binary32; widening appends 16
    zero bits.  Parity: pinned against torch's bfloat16 conversion on all
    65536 patterns.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> float64, from the bit fields.

    sign(1) exponent(4, bias 7) mantissa(3).  Exponent field 0 is
    subnormal: ``m/8 * 2**-6``.  Field 15 with mantissa 7 is NaN; there are
    no infinities.  Parity: pinned against torch.float8_e4m3fn on all 256
    codes and against hand values (1.0, 448, 2**-9).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return sign * mag


def decode_rows(data: np.ndarray, fmt: str, scale: np.ndarray | None,
                rows: np.ndarray) -> np.ndarray:
    """Decode the stored rows ``rows`` of a [rows, ...] tensor to float64.

    ``fmt`` is ``"f32"`` (float32 values), ``"bf16"`` (uint16 bit patterns),
    ``"fp8"`` (uint8 e4m3fn codes; row ``r`` is multiplied by
    ``scale[r // 128]``) or ``"fp8_row"`` (e4m3fn codes; row ``r`` is
    multiplied by its own ``scale[r]``, the format the cache write encodes).
    """
    rows = np.asarray(rows, dtype=np.int64)
    picked = np.asarray(data)[rows]
    if fmt == "f32":
        return picked.astype(np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(picked)
    if fmt == "fp8":
        if scale is None:
            raise ValueError("fp8 rows need a per-block scale")
        vals = e4m3fn_to_f64(picked)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        s = s[rows // FP8_BLOCK_ROWS]
        return vals * s.reshape((-1,) + (1,) * (vals.ndim - 1))
    if fmt == "fp8_row":
        if scale is None:
            raise ValueError("fp8 rows need their per-row scale")
        vals = e4m3fn_to_f64(picked)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)[rows]
        return vals * s.reshape((-1,) + (1,) * (vals.ndim - 1))
    raise ValueError(f"unknown storage format {fmt!r}")


# --------------------------------------------------------------------------
# which physical rows a query's causal keys live in
# --------------------------------------------------------------------------

def contiguous_key_rows(kv_start: int, kv_len: int) -> np.ndarray:
    """Prefill: the reranged KV is in logical order, so the causal keys of a
    query are the rows ``kv_start .. kv_start + kv_len - 1``."""
    return np.arange(kv_start, kv_start + kv_len, dtype=np.int64)


def paged_key_rows(page_table: np.ndarray, page_size: int, req: int,
                   kv_start: int, kv_len: int) -> np.ndarray:
    """Decode: logical position ``p`` of request ``req`` lives in physical row
    ``page_table[req, p // page_size] * page_size + p % page_size``."""
    out = []
    for p in range(kv_start, kv_start + kv_len):
        page = int(page_table[req, p // page_size])
        out.append(page * page_size + p % page_size)
    return np.asarray(out, dtype=np.int64)


# --------------------------------------------------------------------------
# indexer, top-k, sparse MLA
# --------------------------------------------------------------------------

def indexer_scores_row(q_idx_j: np.ndarray, w_j: np.ndarray,
                       keys: np.ndarray) -> np.ndarray:
    """Scores of one query against its causal keys, in key-position order.

    ``q_idx_j`` [h_idx, d_idx], ``w_j`` [h_idx], ``keys`` [L, d_idx] (the
    query's causal indexer keys, position 0 first; all float64).  Returns
    float64 [L]: ``sum_h w_j[h] * max(0, q_idx_j[h] . keys[p])``.
    Parity: pinned (closed-form identity relu(x)-relu(-x)=x, linearity in
    w, hand-worked example, key locality).
    """
    dots = q_idx_j @ keys.T                     # [h_idx, L]
    return w_j @ np.maximum(dots, 0.0)          # [L]


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """Key positions of the ``k`` largest scores; ties go to the lower
    position.  Returns ``min(k, len(scores))`` positions ordered by (score
    descending, position ascending).  Parity: pinned (characterisation by
    brute force, a partition-based second implementation, k >= length).
    """
    scores = np.asarray(scores)
    pos = np.arange(scores.size)
    order = np.lexsort((pos, -scores))          # primary: -score, then pos
    return order[: min(k, scores.size)].astype(np.int64)


def pad_indices(rows: np.ndarray, k: int) -> np.ndarray:
    out = np.full(k, -1, dtype=np.int64)
    out[: rows.size] = rows
    return out


def sparse_mla_row(q_j: np.ndarray, keys: np.ndarray, sm_scale: float,
                   d_latent: int):
    """Latent attention of one query's heads over its selected rows.

    ``q_j`` [H, d_latent + d_rope]; ``keys`` [L, d_latent + d_rope] -- the
    selected latent rows (their order does not matter).  Value = first
    ``d_latent`` columns of each row.  Returns ``(out [H, d_latent],
    lse [H])`` in float64.  Parity: pinned (dense causal attention via
    torch's scaled_dot_product_attention when k covers the context,
    one-key and zero-query closed forms, order invariance).
    """
    if keys.shape[0] == 0:
        return (np.zeros((q_j.shape[0], d_latent)),
                np.full(q_j.shape[0], -np.inf))
    vals = keys[:, :d_latent]                       # [L, d_latent]
    logits = sm_scale * (q_j @ keys.T)              # [H, L]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    den = p.sum(axis=1)
    out = (p @ vals) / den[:, None]
    lse = m[:, 0] + np.log(den)
    return out, lse
