"""GPU parity of kv_cache_write (the rank keeps its own KV in the paged
pool) against oracle/kv_cache.py: bit-exact, on the metadata the split
kernel itself produces."""

import numpy as np
import pytest
import torch

import deepseek_v3_context_amd as ds
from oracle import kv_cache as kc
from oracle import round_robin_cp as rr

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pages(own, page_size, rng, spare=3, holes=False):
    """Random page table for each request's own tokens (a shuffled pool
    with a few spare pages); with holes, every third page is unmapped."""
    counts = [-(-int(c) // page_size) for c in own]
    width = max(counts + [1])
    perm = rng.permutation(sum(counts) + spare).astype(np.int32)
    table = np.full((len(own), width), -1, dtype=np.int32)
    off = 0
    for b, k in enumerate(counts):
        table[b, :k] = perm[off: off + k]
        off += k
    if holes:
        table[:, ::3] = -1
    return table, (sum(counts) + spare) * page_size


def _case(cu, cp, r, row_shape, np_dtype, page_size, seed, holes=False, short_pool=False):
    print(f"[kv_cache_write] cu={list(cu)[:4]}.. cp={cp} r={r} row={row_shape} "
          f"ps={page_size} holes={holes} short={short_pool}", flush=True)
    rng = np.random.default_rng(seed)
    cu = np.asarray(cu, dtype=np.int32)
    T = int(cu[-1])
    meta_h = rr.split_metadata(cu, cp, r)
    own = np.diff(meta_h["local_cu"])
    table, pool_rows = _pages(own, page_size, rng, holes=holes)
    if short_pool:
        pool_rows = max(pool_rows - 2 * page_size - 1, 0)
    full = rng.integers(0, 255, size=(T,) + row_shape, dtype=np.uint8).view(np_dtype) \
        if np_dtype == np.uint8 else rng.integers(0, 1 << 15, size=(T,) + row_shape).astype(np_dtype)
    pool0 = rng.integers(0, 1 << 7, size=(pool_rows,) + row_shape).astype(np_dtype)
    # device side: the split kernel gathers the rank's rows and its metadata
    src = torch.from_numpy(full).to(DEV)
    meta = ds.cp_split_metadata(torch.from_numpy(cu).to(DEV), T, cp, r, rows_src=src)
    pool = torch.from_numpy(pool0).to(DEV)
    ds.kv_cache_write(meta["rows"], meta["batch_idx"], meta["local_cu"],
                      torch.from_numpy(table).to(DEV), page_size, pool)
    got = pool.cpu().numpy()
    # oracle side: its own split of the same rows
    rows_h = rr.split_rows(full, cp, r) if len(meta_h["batch_idx"]) else full[:0]
    want = kc.own_kv_cache_write(rows_h, meta_h["batch_idx"], meta_h["local_cu"], table,
                                 page_size, pool0)
    assert got.shape == want.shape
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    return got, want


@pytest.mark.parametrize("page_size", [1, 16, 64])
@pytest.mark.parametrize("row_shape,np_dtype", [((576,), np.int16), ((128,), np.int16),
                                                ((3,), np.uint8)])
def test_small_batches_every_row(page_size, row_shape, np_dtype):
    _case([0, 37, 41, 130, 200], 4, 2, row_shape, np_dtype, page_size, seed=page_size)


@pytest.mark.parametrize("page_size", [16, 64])
def test_unmapped_pages_and_a_short_pool_leave_the_rest_alone(page_size):
    _case([0, 300, 301, 700], 4, 1, (576,), np.int16, page_size, seed=7, holes=True,
          short_pool=True)


def test_rank_without_tokens_writes_nothing():
    got, want = _case([0, 3], 8, 5, (576,), np.int16, 64, seed=3)
    assert np.array_equal(got, want)


def test_full_size_8000_token_prefill_rank0():
    _case([0, 8000], 8, 0, (576,), np.int16, 64, seed=11)


def test_full_size_65536_token_prefill_rank3_and_indexer_keys():
    _case([0, 65536], 8, 3, (576,), np.int16, 64, seed=12)
    _case([0, 65536], 8, 3, (128,), np.uint8, 64, seed=13)   # fp8 indexer keys: 128 B rows


def test_six_requests_25305_tokens_rank5():
    cu = [0, 1000, 5000, 5001, 12000, 20000, 25305]
    _case(cu, 8, 5, (576,), np.int16, 64, seed=14)


# ------------------------------------------------------------ prefill -> decode

@pytest.mark.parametrize("name", ["small_decode_paged", "small_decode_paged_fp8"])
def test_decode_reads_what_the_prefill_rank_kept(name):
    """The decode path on a pool that kv_cache_write filled from each
    request's rows in logical order (a cp 1 prefill keeps every token): the
    pool matches the drawn one at every mapped row and is untouched
    elsewhere, and decode output passes the decode parity gates.  For the
    fp8 workload this is a byte-permutation check: the codes are moved as
    given and keep the pool's own per-128-row scales (the fp8 encoding on
    write, with a scale per row, is checked below)."""
    from synth import draw_decode, get
    from oracle import pipeline as opl
    from tests import gpu_path as gp
    from tests import test_gpu_parity as tgp

    wl = get(name)
    inp = draw_decode(wl)
    print(f"[kv_cache_write -> decode] {name}", flush=True)
    lengths = inp["lengths"].astype(np.int64)
    table, ps = inp["page_table"], wl.page_size
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    phys = np.concatenate([sa_rows(table, ps, b, int(L)) for b, L in enumerate(lengths)])
    meta = None
    pools = {}
    for key in ("kv", "k_idx"):
        drawn = np.ascontiguousarray(inp[key])
        nrow = drawn.shape[0]
        as_bytes = drawn.reshape(nrow, -1).view(np.uint8)          # rows as raw bytes
        logical = torch.from_numpy(np.ascontiguousarray(as_bytes[phys])).to(DEV)
        meta = ds.cp_split_metadata(torch.from_numpy(cu).to(DEV), T, 1, 0, rows_src=logical)
        # all-ones bytes: NaN in bf16 and in e4m3fn, so a read of an unwritten row shows
        pool = torch.full(as_bytes.shape, 0xFF, dtype=torch.uint8, device=DEV)
        ds.kv_cache_write(meta["rows"], meta["batch_idx"], meta["local_cu"],
                          torch.from_numpy(table).to(DEV), ps, pool)
        got = pool.cpu().numpy()
        mapped = np.zeros(nrow, bool)
        mapped[phys] = True
        assert np.array_equal(got[mapped], as_bytes[mapped])
        assert (got[~mapped] == 0xFF).all()
        pools[key] = got.view(drawn.dtype).reshape(drawn.shape)
    inp2 = dict(inp, kv=pools["kv"], k_idx=pools["k_idx"])
    g = gp.run_decode(wl, inp2)
    dmeta = opl.decode_metadata(inp["lengths"])
    rows = list(range(wl.n_req))
    sel = opl.indexer_topk_rows(rows, dmeta, inp["q_idx"], wl.act_fmt, inp["w"], inp["k_idx"],
                                wl.kv_fmt, inp["k_idx_scale"], wl.topk,
                                page_table=table, page_size=ps)
    tgp._check_rows(wl, g, sel, rows, inp, inp["kv"], inp["kv_scale"])


def sa_rows(table, page_size, b, L):
    """Physical pool rows of request b's positions 0..L-1 (test-side data
    preparation: the decode pool layout the workload generator drew)."""
    p = np.arange(L)
    return table[b, p // page_size].astype(np.int64) * page_size + p % page_size


# ------------------------------------------------------------ fp8 on write

def _fp8_case(cu, cp, r, D, page_size, seed, holes=False, short_pool=False, planted=False,
              spread=True):
    """The rank's own bf16 rows (gathered by the split kernel) encoded into
    an fp8 pool with a scale per row: codes and scales bit-exact against
    the oracle, unmapped rows untouched."""
    print(f"[kv_cache_write_fp8] cu={list(cu)[:4]}.. cp={cp} r={r} D={D} ps={page_size}",
          flush=True)
    from synth.draw import to_bf16_bits
    rng = np.random.default_rng(seed)
    cu = np.asarray(cu, dtype=np.int32)
    T = int(cu[-1])
    meta_h = rr.split_metadata(cu, cp, r)
    own = np.diff(meta_h["local_cu"])
    table, pool_rows = _pages(own, page_size, rng, holes=holes)
    if short_pool:
        pool_rows = max(pool_rows - 2 * page_size - 1, 0)
    # spread: row magnitudes over five decades (the scale per row follows
    # them); else the workloads' N(0,1)/sqrt(D) activations
    mag = rng.uniform(1e-3, 30.0, (T, 1)) if spread else D ** -0.5
    x = (rng.standard_normal((T, D)) * mag).astype(np.float32)
    if planted:
        # rows whose scale is exactly 1 (amax 448) and whose other values are
        # e4m3fn midpoints (ties), negative values, tiny values, zeros
        from oracle.sparse_attention import e4m3fn_to_f64
        vals = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
        mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
        for t in range(min(T, 40)):
            row = rng.choice(np.concatenate([mids, -mids, vals[:20], -vals[:20]]), D)
            row[t % D] = 448.0
            x[t] = row
        x[40:48] = 0.0                                            # all-zero rows (every rank)
    full = to_bf16_bits(x)
    src = torch.from_numpy(full.view(np.int16)).to(DEV).view(torch.bfloat16)
    meta = ds.cp_split_metadata(torch.from_numpy(cu).to(DEV), T, cp, r, rows_src=src)
    codes0 = np.full((pool_rows, D), 0x7F, dtype=np.uint8)
    scale0 = np.full(pool_rows, -1.0, dtype=np.float32)
    codes = torch.from_numpy(codes0).to(DEV)
    scales = torch.from_numpy(scale0).to(DEV)
    ds.kv_cache_write_fp8(meta["rows"], meta["batch_idx"], meta["local_cu"],
                          torch.from_numpy(table).to(DEV), page_size, codes, scales)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    rows_h = rr.split_rows(full, cp, r) if len(meta_h["batch_idx"]) else full[:0]
    want_c, want_s = kc.own_kv_cache_write_fp8(rows_h, meta_h["batch_idx"], meta_h["local_cu"],
                                               table, page_size, codes0, scale0)
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    return table, pool_rows, got_c, got_s, full, meta_h


@pytest.mark.parametrize("D", [576, 128, 4, 1024])
@pytest.mark.parametrize("page_size", [1, 64])
def test_fp8_write_small_batches_bit_exact(D, page_size):
    _fp8_case([0, 37, 41, 130, 200], 4, 2, D, page_size, seed=20 + D + page_size, planted=True)


def test_fp8_write_unmapped_pages_and_short_pool():
    _fp8_case([0, 300, 301, 700], 4, 1, 576, 16, seed=31, holes=True, short_pool=True)


def test_fp8_write_full_size_65536_token_rank3():
    _fp8_case([0, 65536], 8, 3, 576, 64, seed=32)
    _fp8_case([0, 65536], 8, 3, 128, 64, seed=33)


@pytest.mark.parametrize("heads", [128, 64])
def test_fp8_written_pool_read_back_by_decode(heads):
    """Prefill -> decode in fp8: a rank's own latent rows and indexer keys
    (bf16, from a three-request prefill) encoded into fp8 pools with a scale
    per row; then one decode query per request over the rank's cache
    (indexer + top-k on the paged keys, sparse MLA decode and prefill on the
    paged latent rows, all reading the per-row scales) against the oracle
    on the same codes and scales."""
    from oracle import pipeline as opl
    from synth.draw import to_bf16_bits
    from tests import gpu_path as gp
    from tests import test_gpu_parity as tgp

    cu, cp, r, ps, topk = [0, 1900, 3300, 3340], 4, 1, 64, 256
    t_lat = _fp8_case(cu, cp, r, 576, ps, seed=40 + heads, spread=False)
    table, pool_rows, kv_c, kv_s, _, meta_h = t_lat
    # the indexer keys share the latent pool's page table
    rng = np.random.default_rng(50 + heads)
    T = cu[-1]
    xk = (rng.standard_normal((T, 128)) / np.sqrt(128)).astype(np.float32)
    fk = to_bf16_bits(xk)
    srck = torch.from_numpy(fk.view(np.int16)).to(DEV).view(torch.bfloat16)
    meta = ds.cp_split_metadata(torch.tensor(cu, dtype=torch.int32, device=DEV), T, cp, r,
                                rows_src=srck)
    ki_c = torch.full((pool_rows, 128), 0x7F, dtype=torch.uint8, device=DEV)
    ki_s = torch.full((pool_rows,), -1.0, dtype=torch.float32, device=DEV)
    ds.kv_cache_write_fp8(meta["rows"], meta["batch_idx"], meta["local_cu"],
                          torch.from_numpy(table).to(DEV), ps, ki_c, ki_s)
    lengths = np.diff(meta_h["local_cu"]).astype(np.int32)       # the rank's cache per request
    n = lengths.size
    q_idx = to_bf16_bits((rng.standard_normal((n, 64, 128)) / np.sqrt(128)).astype(np.float32))
    w = (rng.standard_normal((n, 64)) / 8).astype(np.float32)
    q = to_bf16_bits((rng.standard_normal((n, heads, 576)) / 24).astype(np.float32))
    dm = ds.decode_metadata(torch.from_numpy(lengths).to(DEV))
    paging = dict(q_req=dm["q_req"], page_table=torch.from_numpy(table).to(DEV), page_size=ps)
    kd = ki_c.view(torch.float8_e4m3fn)
    idx, score = ds.indexer_topk(gp.to_dev(q_idx, "bf16"), torch.from_numpy(w).to(DEV), kd,
                                 dm["kv_start"], dm["kv_len"], int(lengths.max()), topk,
                                 k_scale=ki_s, want_score=True, scale_per_row=True, **paging)
    sc = ds.indexer_scores(gp.to_dev(q_idx, "bf16"), torch.from_numpy(w).to(DEV), kd,
                           dm["kv_start"], dm["kv_len"], int(lengths.max()), k_scale=ki_s,
                           scale_per_row=True, **paging)
    kvd = torch.from_numpy(kv_c).to(DEV).view(torch.float8_e4m3fn)
    kvs = torch.from_numpy(kv_s).to(DEV)
    qd = gp.to_dev(q, "bf16")
    out_d, lse_d = ds.sparse_mla_decode(qd, kvd, idx, 1 / 24, 512, kv_scale=kvs, scale_per_row=True)
    out_p, lse_p = ds.sparse_mla_prefill(qd, kvd, idx, 1 / 24, 512, kv_scale=kvs, scale_per_row=True)
    torch.cuda.synchronize()
    g = {"scores": sc.cpu().numpy(), "topk_idx": idx.cpu().numpy(), "topk_score": score.cpu().numpy(),
         "out": out_d.float().cpu().numpy(), "lse": lse_d.cpu().numpy(),
         "out_prefill_kernel": out_p.float().cpu().numpy(), "lse_prefill_kernel": lse_p.cpu().numpy()}

    from types import SimpleNamespace
    W = SimpleNamespace(kind="decode", topk=topk, act_fmt="bf16", kv_fmt="fp8_row", scale=1 / 24,
                        d_latent=512, name=f"fp8 pool {heads}h")   # the parity helper's workload view
    meta_d = {"q_req": np.arange(n, dtype=np.int32), "kv_start": np.zeros(n, np.int32),
              "kv_len": lengths}
    rows = list(range(n))
    sel = opl.indexer_topk_rows(rows, meta_d, q_idx, "bf16", w, ki_c.cpu().numpy(), "fp8_row",
                                ki_s.cpu().numpy(), topk, page_table=table, page_size=ps)
    tgp._check_rows(W, g, sel, rows, {"q": q}, kv_c, kv_s)
