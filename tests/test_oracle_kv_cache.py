"""Pins of oracle/kv_cache.py (own-KV retention in the paged pool)."""

import numpy as np
import pytest
import torch

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


# ------------------------------------------------ fp8 encoding of the kept rows

from oracle.sparse_attention import e4m3fn_to_f64  # noqa: E402


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_e4m3fn_encoder_matches_torch_on_values_midpoints_and_random():
    vals = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2          # ties: round to the even code
    rnd = np.random.default_rng(3).uniform(-448, 448, 20000)
    small = np.random.default_rng(4).uniform(-2 ** -5, 2 ** -5, 5000)   # subnormal range
    x = np.concatenate([vals, -vals, mids, -mids, rnd, small])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kc.encode_e4m3fn(x), ref)


def test_e4m3fn_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(kc.encode_e4m3fn(e4m3fn_to_f64(codes)), codes)   # -0 -> 0x80 too
    with pytest.raises(ValueError):
        kc.encode_e4m3fn([449.0])


def test_row_encoding_hand_example():
    # amax 1.0 -> scale 1/448; 1.0 -> 448 (0x7E), -0.5 -> -224 (1.75 * 2^7:
    # 0xF6), 0.25 -> 112 (1.75 * 2^6: 0x6E), 0 -> 0
    codes, scale = kc.encode_row_fp8(_bf16([1.0, -0.5, 0.25, 0.0]))
    assert scale == np.float32(1.0) / np.float32(448.0)
    assert codes.tolist() == [0x7E, 0xF6, 0x6E, 0x00]
    z_codes, z_scale = kc.encode_row_fp8(_bf16([0.0] * 8))
    assert z_scale == 0 and not z_codes.any()


def test_row_encoding_error_bound_and_amax_code():
    rng = np.random.default_rng(9)
    for row in rng.standard_normal((50, 576)).astype(np.float32) * rng.uniform(1e-3, 1e3, (50, 1)):
        b = _bf16(row)
        x = b.astype(np.uint32) << 16
        x = x.view(np.float32).astype(np.float64)
        codes, scale = kc.encode_row_fp8(b)
        back = e4m3fn_to_f64(codes) * np.float64(scale)
        # nearest of 3 mantissa bits: relative half-ulp 2^-4 for normals, an
        # absolute half-step scale * 2^-10 in the subnormal range; plus the
        # float32 rounding of x / scale
        assert np.all(np.abs(back - x) <= 2 ** -4 * np.abs(x) * (1 + 1e-6) + float(scale) * 2 ** -10)
        assert np.abs(e4m3fn_to_f64(codes)).max() == 448.0      # the amax element


def test_fp8_write_lands_where_the_plain_write_does():
    rng = np.random.default_rng(12)
    n_req, ps = 3, 4
    counts = [5, 0, 9]
    batch_idx = np.repeat(np.arange(n_req), counts).astype(np.int32)
    local_cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    table = np.array([[3, 0, -1], [-1, -1, -1], [5, 1, 7]], dtype=np.int32)   # page 7 past the pool
    pool_rows = 7 * ps
    rows = _bf16(rng.standard_normal((len(batch_idx), 16)))
    codes0 = np.full((pool_rows, 16), 0x7F, dtype=np.uint8)                    # NaN where unwritten
    scale0 = np.full(pool_rows, -1.0, dtype=np.float32)
    codes, scales = kc.own_kv_cache_write_fp8(rows, batch_idx, local_cu, table, ps, codes0, scale0)
    marker = np.arange(len(batch_idx), dtype=np.int64)[:, None] * np.ones((1, 16), np.int64)
    placed = kc.own_kv_cache_write(marker, batch_idx, local_cu, table, ps,
                                   np.full((pool_rows, 16), -1, dtype=np.int64))
    for r in range(pool_rows):
        j = placed[r, 0]
        if j < 0:
            assert (codes[r] == 0x7F).all() and scales[r] == -1.0
        else:
            want_c, want_s = kc.encode_row_fp8(rows[j])
            assert np.array_equal(codes[r], want_c) and scales[r] == want_s
    assert (placed[:, 0] >= 0).sum() == 5 + 8     # request 2's last row maps to page 7: dropped


def test_per_row_scale_decoding_agrees_with_the_block_decoding():
    # a per-row scale array that repeats each 128-row block's scale decodes
    # every row exactly as the per-block format does
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 256, size=(300, 8), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                 # no NaN codes
    blk = rng.uniform(0.01, 2.0, 3).astype(np.float32)
    per_row = np.repeat(blk, 128)[:300]
    rows = rng.permutation(300)[:100]
    assert np.array_equal(sa.decode_rows(codes, "fp8_row", per_row, rows),
                          sa.decode_rows(codes, "fp8", blk, rows))
