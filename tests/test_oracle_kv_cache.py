"""Pins of oracle/kv_cache.py (own-KV retention in the paged pool)."""

import numpy as np

from oracle import kv_cache as kc
from oracle import round_robin_cp as rr
from oracle import sparse_attention as sa


def _meta(cu, cp, r):
    m = rr.split_metadata(np.asarray(cu), cp, r)
    return m["batch_idx"], m["local_cu"]


def test_page_example_rank1_keeps_its_own_tokens():
    # the page's 8-token example on 4 ranks: rank 1 owns T1 and T5, which
    # are its cache positions 0 and 1 (one request)
    bi, lcu = _meta([0, 8], 4, 1)
    assert list(bi) == [0, 0] and list(lcu) == [0, 2]
    assert kc.own_cache_position(0, bi, lcu) == (0, 0)
    assert kc.own_cache_position(1, bi, lcu) == (0, 1)
    rows = np.array([[11], [55]], dtype=np.int32)          # K1, K5
    pool = np.full((8, 1), -7, dtype=np.int32)
    table = np.array([[3, 1]], dtype=np.int32)              # page size 2: rows 6, 7 first
    out = kc.own_kv_cache_write(rows, bi, lcu, table, 2, pool)
    assert out[6, 0] == 11 and out[7, 0] == 55
    assert (np.delete(out[:, 0], [6, 7]) == -7).all()


def test_hand_worked_two_requests():
    # cu_seqlens [0, 5, 8] on cp 2, rank 1: global tokens 1, 3 (request 0)
    # and 5, 7 (request 1); local_cu [0, 2, 4]
    bi, lcu = _meta([0, 5, 8], 2, 1)
    assert list(bi) == [0, 0, 1, 1] and list(lcu) == [0, 2, 4]
    rows = np.array([[1, 1], [3, 3], [5, 5], [7, 7]], dtype=np.uint8)
    pool = np.zeros((12, 2), dtype=np.uint8)
    # page size 2; request 0 -> page 3 (rows 6, 7); request 1 -> page 0 (rows 0, 1)
    table = np.array([[3, -1], [0, 5]], dtype=np.int32)
    out = kc.own_kv_cache_write(rows, bi, lcu, table, 2, pool)
    expect = np.zeros((12, 2), dtype=np.uint8)
    expect[6] = 1
    expect[7] = 3
    expect[0] = 5
    expect[1] = 7
    assert (out == expect).all()
    assert (pool == 0).all()   # the input pool is not modified


def test_unmapped_pages_and_rows_past_the_pool_are_dropped():
    bi, lcu = _meta([0, 12], 1, 0)                    # one request, 12 own tokens
    rows = np.arange(12, dtype=np.int64).reshape(12, 1) + 100
    pool = np.full((10, 1), -1, dtype=np.int64)
    # page size 4: page 0 -> 0 (rows 0-3), page 1 unmapped, page 2 -> 2 (rows 8-11, only 8, 9 exist)
    table = np.array([[0, -1, 2]], dtype=np.int32)
    out = kc.own_kv_cache_write(rows, bi, lcu, table, 4, pool)
    assert list(out[:, 0]) == [100, 101, 102, 103, -1, -1, -1, -1, 108, 109]
    # a table narrower than the request: positions past it are dropped too
    out2 = kc.own_kv_cache_write(rows, bi, lcu, table[:, :1], 4, pool)
    assert list(out2[:, 0]) == [100, 101, 102, 103] + [-1] * 6


def test_decode_reads_back_what_the_prefill_rank_kept():
    # every own token written through the page table reads back, in order,
    # through the decode path's paged row mapping
    rng = np.random.default_rng(5)
    cu = np.array([0, 37, 41, 130, 200])
    cp, r, ps = 4, 2, 8
    bi, lcu = _meta(cu, cp, r)
    n = len(bi)
    own = np.diff(lcu)
    pages = [-(-int(c) // ps) for c in own]
    perm = rng.permutation(sum(pages) + 3).astype(np.int32)
    table = np.full((len(own), max(pages)), -1, dtype=np.int32)
    off = 0
    for b, k in enumerate(pages):
        table[b, :k] = perm[off: off + k]
        off += k
    rows = rng.integers(0, 1 << 30, size=(n, 3)).astype(np.int64)
    pool = np.zeros((len(perm) * ps, 3), dtype=np.int64)
    out = kc.own_kv_cache_write(rows, bi, lcu, table, ps, pool)
    for b in range(len(own)):
        phys = sa.paged_key_rows(table, ps, b, 0, int(own[b]))
        assert (out[phys] == rows[lcu[b]: lcu[b + 1]]).all()
    # and nothing else was written
    written = np.zeros(len(pool), bool)
    for b in range(len(own)):
        written[sa.paged_key_rows(table, ps, b, 0, int(own[b]))] = True
    assert (out[~written] == 0).all()
