"""Round-robin token split, per-rank metadata and KV rerange -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Everything here is
integer bookkeeping written as plain enumeration over token indices, so that
a reader can check it against the pages by eye.

Sources:

* "[DeepSeek v3.2] 上下文并行详解", section 1 and section 2B: in the
  round-robin mode a token whose index in the flattened batch is ``g`` goes
  to rank ``g mod cp_size``; each rank keeps its own tokens in increasing
  index order; per-rank sequence lengths, batch indices and cumulative
  sequence offsets are recomputed after the split.
* same page, section 4 part 3, step 1 (8 tokens on 4 ranks: rank 0 holds
  T0,T4; rank 1 T1,T5; rank 2 T2,T6; rank 3 T3,T7) and its remark that the
  per-rank token counts never differ by more than one, whatever the batch.
* same page, section 4 part 3, step B: after the all-gather the KV rows sit
  in rank-concatenated order (T0,T4,T1,T5,...) and are put back into
  logical order T0,T1,T2,... (the rerange).
* same page, section 4 part 3, step C, and the causal example there (T5
  attends to T0..T4): a query at position ``p`` of its request sees the keys
  at positions ``0..p`` of the same request (inclusive of itself).
* same page, section 4 part 1: the older contiguous split ("in-seq-split")
  of an 8000-token prompt over 8 ranks, 1000 consecutive tokens each.

Readings taken where the pages are silent (listed again in the design doc):

* the split runs over the flattened global token index of the whole batch,
  not per request (the page's split indexes the total token count and its
  balance claim holds for any number of requests);
* the all-gather delivers equal slots of ``slot_rows`` rows per rank, rank
  after rank; rows past a rank's count are padding and are never read.
"""

from __future__ import annotations

import numpy as np


def owner_rank(g: int, cp_size: int) -> int:
    """Rank that owns global token ``g`` under the round-robin split."""
    return g % cp_size


def rank_global_ids(num_tokens: int, cp_size: int, cp_rank: int) -> np.ndarray:
    """Global token indices owned by ``cp_rank``, in increasing order.

    Plain enumeration: walk every token and keep those the rank owns.
    """
    _check_rank(cp_size, cp_rank)
    kept = [g for g in range(num_tokens) if owner_rank(g, cp_size) == cp_rank]
    return np.asarray(kept, dtype=np.int64)


def local_count(num_tokens: int, cp_size: int, cp_rank: int) -> int:
    """Number of tokens rank ``cp_rank`` owns (by enumeration)."""
    return int(rank_global_ids(num_tokens, cp_size, cp_rank).size)


def split_metadata(cu_seqlens, cp_size: int, cp_rank: int) -> dict:
    """Per-rank metadata after the round-robin split.

    ``cu_seqlens`` is the batch's cumulative sequence offsets ``[B+1]``
    (``cu[0] = 0``, request ``b`` owns global tokens ``cu[b] .. cu[b+1]-1``).

    Returns int32 arrays:

    * ``global_idx[j]`` -- global token index of the rank's j-th query;
    * ``batch_idx[j]``  -- request that token belongs to;
    * ``local_cu[b]``   -- number of the rank's tokens with global index
      below ``cu[b]`` (the recomputed cumulative offsets of the rank's
      shortened sequences);
    * ``kv_start[j]``   -- first global KV row of the query's request;
    * ``kv_len[j]``     -- number of causal keys: positions ``0..p`` where
      ``p`` is the query's position within its request.

    Parity: pinned (tests/test_oracle_round_robin.py).
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    num_tokens = cu[-1]
    gids = rank_global_ids(num_tokens, cp_size, cp_rank)

    batch_idx = []
    for g in gids.tolist():
        owner = None
        for b in range(len(cu) - 1):
            if cu[b] <= g < cu[b + 1]:
                owner = b
                break
        assert owner is not None
        batch_idx.append(owner)

    local_cu = []
    for bound in cu:
        local_cu.append(sum(1 for g in gids.tolist() if g < bound))

    kv_start = [cu[b] for b in batch_idx]
    kv_len = [g - s + 1 for g, s in zip(gids.tolist(), kv_start)]
    as32 = lambda v: np.asarray(v, dtype=np.int32).reshape(-1)  # noqa: E731
    return {
        "global_idx": as32(gids),
        "batch_idx": as32(batch_idx),
        "local_cu": as32(local_cu),
        "kv_start": as32(kv_start),
        "kv_len": as32(kv_len),
    }


def split_rows(x: np.ndarray, cp_size: int, cp_rank: int) -> np.ndarray:
    """Rows of ``x`` (first axis = global token) that ``cp_rank`` keeps."""
    ids = np.arange(x.shape[0])
    keep = (ids % cp_size) == cp_rank
    return x[keep]


def rank_concat(x: np.ndarray, cp_size: int, slot_rows: int | None = None,
                pad_value=None) -> np.ndarray:
    """What an all-gather of each rank's own rows delivers.

    Slot ``r`` (rows ``r*slot_rows .. (r+1)*slot_rows-1``) holds
    ``split_rows(x, cp_size, r)`` followed by padding.  ``slot_rows``
    defaults to the largest per-rank count.  Padding rows are filled with
    ``pad_value`` (default: NaN for floating dtypes, all-ones bytes
    otherwise) so that a reader of padding is visible.
    """
    num_tokens = x.shape[0]
    counts = [local_count(num_tokens, cp_size, r) for r in range(cp_size)]
    if slot_rows is None:
        slot_rows = max(counts) if counts else 0
    if slot_rows < max(counts):
        raise ValueError("slot_rows smaller than a rank's token count")
    out = np.empty((cp_size * slot_rows,) + x.shape[1:], dtype=x.dtype)
    if pad_value is None:
        if np.issubdtype(x.dtype, np.floating):
            out.fill(np.nan)
        else:
            out.view(np.uint8).fill(0xFF)
    else:
        out.fill(pad_value)
    for r in range(cp_size):
        mine = split_rows(x, cp_size, r)
        out[r * slot_rows: r * slot_rows + mine.shape[0]] = mine
    return out


def rerange(concat: np.ndarray, num_tokens: int, cp_size: int,
            slot_rows: int) -> np.ndarray:
    """Put rank-concatenated rows back into logical token order.

    Written in scatter form, rank by rank: the j-th row of rank ``r``'s slot
    is global token ``r + j*cp_size``.  Parity: pinned.
    """
    if concat.shape[0] < cp_size * slot_rows:
        raise ValueError("concat buffer shorter than cp_size * slot_rows")
    out = np.empty((num_tokens,) + concat.shape[1:], dtype=concat.dtype)
    written = np.zeros(num_tokens, dtype=bool)
    for r in range(cp_size):
        j = 0
        while True:
            g = r + j * cp_size
            if g >= num_tokens:
                break
            if j >= slot_rows:
                raise ValueError("rank slot too small for its tokens")
            out[g] = concat[r * slot_rows + j]
            written[g] = True
            j += 1
    assert written.all()
    return out


def in_seq_split_ranges(num_tokens: int, cp_size: int) -> list[tuple[int, int]]:
    """Contrast mode: the older contiguous split (inclusive ranges).

    Section 4 part 1 of the blog post: each rank takes one contiguous chunk
    of ``ceil(T / cp_size)`` tokens.  Used only to pin the page's 8000-token
    example; not on the hot path.
    """
    chunk = -(-num_tokens // cp_size)
    out = []
    for r in range(cp_size):
        lo = r * chunk
        hi = min(num_tokens, lo + chunk) - 1
        out.append((lo, hi))
    return out


def in_seq_split_metadata(cu_seqlens, cp_size: int, cp_rank: int) -> dict:
    """Contrast mode: per-rank metadata under the older contiguous split.

    Section 4 part 1 of the blog post: each request is cut into ``cp_size``
    consecutive chunks and rank ``r`` takes chunk ``r`` of every request (an
    8000-token prompt on 8 ranks: rank 0 tokens 0..999, rank 1 1000..1999;
    with a second, 800-token request rank 0 also takes its tokens 0..99).
    Reading taken where the page is silent: a request of ``L`` tokens is
    cut into chunks of ``ceil(L / cp_size)`` tokens (the last chunks may be
    shorter or empty), at token granularity.

    Written as plain enumeration: walk every token of every request, find
    its chunk, keep it if the chunk is this rank's.  Same fields as
    :func:`split_metadata`; ``kv_len`` is again position + 1 within the
    request (causal).  Parity: pinned (tests/test_oracle_round_robin.py).
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    _check_rank(cp_size, cp_rank)
    gids, batch_idx, kv_start, kv_len, local_cu = [], [], [], [], [0]
    for b in range(len(cu) - 1):
        length = cu[b + 1] - cu[b]
        chunk = -(-length // cp_size)
        for p in range(length):
            if p // chunk == cp_rank:
                gids.append(cu[b] + p)
                batch_idx.append(b)
                kv_start.append(cu[b])
                kv_len.append(p + 1)
        local_cu.append(len(gids))
    as32 = lambda v: np.asarray(v, dtype=np.int32).reshape(-1)  # noqa: E731
    return {
        "global_idx": as32(gids),
        "batch_idx": as32(batch_idx),
        "local_cu": as32(local_cu),
        "kv_start": as32(kv_start),
        "kv_len": as32(kv_len),
    }


def _check_rank(cp_size: int, cp_rank: int) -> None:
    if cp_size < 1 or not (0 <= cp_rank < cp_size):
        raise ValueError(f"bad cp_size/cp_rank {cp_size}/{cp_rank}")
