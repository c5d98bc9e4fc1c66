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
  the rows; no re-encoding).
"""

from __future__ import annotations

import numpy as np


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
