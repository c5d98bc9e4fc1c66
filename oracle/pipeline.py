"""One rank's hot path, step by step, for chosen query rows -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Chains the plain
definitions of :mod:`oracle.round_robin_cp` and
:mod:`oracle.sparse_attention` in the order the blog post's section 4 part 3
gives them: split (step 1), gather + rerange of KV (step B), then local
queries against the complete KV (step C) -- indexer scores, top-k, sparse
latent attention.  Rows are processed one query at a time so that any
subset of a large workload can be checked.

The top-k decision is taken on the scores rounded to float32, the precision
in which the device path stores and compares them; entries whose float64
score lies within a small band of the k-th score may legitimately differ
between two correct implementations and are compared with that band.
"""

from __future__ import annotations

import numpy as np

from . import round_robin_cp as rr
from . import sparse_attention as sa


def decode_metadata(lengths) -> dict:
    """Decode step: request ``i`` has one query at position ``L_i - 1``; its
    own KV is already in the cache, so its causal keys are positions
    ``0 .. L_i - 1`` of that request."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return {"q_req": np.arange(lengths.size, dtype=np.int32),
            "kv_start": np.zeros(lengths.size, dtype=np.int32),
            "kv_len": lengths.astype(np.int32)}


def key_rows_for(j: int, meta: dict, page_table=None, page_size=None):
    start, length = int(meta["kv_start"][j]), int(meta["kv_len"][j])
    if page_table is None:
        return sa.contiguous_key_rows(start, length)
    req = int(meta["q_req"][j])
    return sa.paged_key_rows(page_table, page_size, req, start, length)


def indexer_topk_rows(rows, meta, q_idx, q_fmt, w, k_idx, k_fmt, k_scale,
                      topk, page_table=None, page_size=None):
    """Indexer scores and top-k for the query rows ``rows``.

    Returns a list of dicts, one per row: ``key_rows`` (physical rows of the
    causal keys in position order), ``scores64`` (float64), ``scores32``
    (rounded to float32), ``sel_pos`` (selected positions, best first) and
    ``topk_idx`` (physical rows, -1 padded to ``topk``).
    """
    out = []
    for j in rows:
        j = int(j)
        krows = key_rows_for(j, meta, page_table, page_size)
        keys = sa.decode_rows(k_idx, k_fmt, k_scale, krows)
        qj = sa.decode_rows(q_idx, q_fmt, None, [j])[0]
        wj = np.asarray(w[j], dtype=np.float32).astype(np.float64)
        s64 = sa.indexer_scores_row(qj, wj, keys)
        s32 = s64.astype(np.float32)
        pos = sa.topk_positions(s32, topk)
        out.append({"key_rows": krows, "scores64": s64, "scores32": s32,
                    "sel_pos": pos,
                    "topk_idx": sa.pad_indices(krows[pos], topk)})
    return out


def sparse_mla_rows(rows, idx, q, q_fmt, kv, kv_fmt, kv_scale, sm_scale,
                    d_latent):
    """Sparse latent attention for query rows ``rows``; ``idx[i]`` holds the
    physical KV rows selected for ``rows[i]`` (-1 = empty slot).  Returns
    ``(out [len(rows), H, d_latent], lse [len(rows), H])`` in float64."""
    outs, lses = [], []
    for i, j in enumerate(rows):
        sel = np.asarray(idx[i])
        sel = sel[sel >= 0]
        keys = sa.decode_rows(kv, kv_fmt, kv_scale, sel)
        qj = sa.decode_rows(q, q_fmt, None, [int(j)])[0]
        o, l = sa.sparse_mla_row(qj, keys, sm_scale, d_latent)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def prefill_rank(cu_seqlens, cp_size, cp_rank):
    """Metadata of one rank (step 1)."""
    return rr.split_metadata(cu_seqlens, cp_size, cp_rank)
