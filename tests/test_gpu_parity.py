"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Gates (written out here, derived in the design doc):

* split metadata, row gather, rank-concatenated buffer and rerange:
  bit-exact;
* indexer scores: |gpu - oracle64| <= 5e-5 (fp32 accumulation of bf16
  products; scores are O(0.1)) and positions past kv_len never written;
* top-k: same count, no duplicates, every index causal, and every element of
  the symmetric difference has an oracle score within 1e-3 of the oracle's
  k-th score; rows with at most k causal keys select exactly all of them;
* sparse MLA, on the GPU's own top-k set: max-abs <= 2e-2 (bf16 KV) or
  6e-2 (fp8 KV), and relative max-abs <= 1e-2 (bf16) / 3e-2 (fp8); fp32
  inputs: max-abs <= 1e-4; lse within 1e-3.

Small workloads are checked on every query row; the full-size ones (the
launch configuration bench.py times) on sampled rows: the first and last
four, 24 seeded random rows, and the first and last local row of every
request.
"""

import numpy as np
import pytest
import torch

from oracle import pipeline as opl
from oracle import round_robin_cp as orr
from oracle import sparse_attention as sa
from synth import draw_decode, draw_prefill, get

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import deepseek_v3_context_amd as ds  # noqa: E402
    from tests import gpu_path as gp  # noqa: E402

SCORE_ATOL = 5e-5
TOPK_BAND = 1e-3


def _sample_rows(n, seed, local_cu=None):
    """First and last four rows, 24 seeded random rows, and the first and
    last local row of every request (local_cu: the rank's request offsets)."""
    if n <= 64:
        return list(range(n))
    rng = np.random.default_rng(seed)
    pick = set(range(4)) | set(range(n - 4, n)) | set(rng.choice(n, 24, replace=False).tolist())
    if local_cu is not None:
        for lo, hi in zip(local_cu[:-1], local_cu[1:]):
            if hi > lo:
                pick |= {int(lo), int(hi) - 1}
    return sorted(pick)


def _mla_gate(wl):
    if wl.kv_fmt == "f32":
        return 1e-4, 1e-4
    if wl.kv_fmt in ("fp8", "fp8_row"):
        return 6e-2, 3e-2
    return 2e-2, 1e-2


def _check_rows(wl, g, orc_sel, rows, inp, kv_data, kv_scale):
    kth_misses = 0
    gidx_rows = []
    for i, (j, s) in enumerate(zip(rows, orc_sel)):
        L = s["key_rows"].size
        # ---- S3 scores
        sc = g["scores"][j]
        assert np.all(np.abs(sc[:L] - s["scores64"]) <= SCORE_ATOL), \
            f"row {j}: score err {np.abs(sc[:L] - s['scores64']).max():.3e}"
        assert np.all(np.isnan(sc[L:])), f"row {j}: wrote past kv_len"
        # ---- S4 top-k
        gi = g["topk_idx"][j]
        valid = gi[gi >= 0]
        assert (gi[valid.size:] == -1).all(), f"row {j}: -1 padding not at the end"
        assert valid.size == min(wl.topk, L), f"row {j}: count {valid.size} vs {min(wl.topk, L)}"
        assert np.unique(valid).size == valid.size, f"row {j}: duplicate indices"
        if wl.kind == "prefill":   # selections come out in ascending key position
            assert (np.diff(valid) > 0).all(), f"row {j}: not in position order"
        pos_of = {int(x): p for p, x in enumerate(s["key_rows"].tolist())}
        assert all(int(x) in pos_of for x in valid), f"row {j}: non-causal index"
        o = s["topk_idx"][s["topk_idx"] >= 0]
        diff = set(valid.tolist()) ^ set(o.tolist())
        if L <= wl.topk:
            assert not diff, f"row {j}: must select every causal key"
        else:
            kth = s["scores64"][s["sel_pos"][-1]]
            far = [x for x in diff if abs(s["scores64"][pos_of[x]] - kth) > TOPK_BAND]
            assert not far, f"row {j}: {len(far)} selections outside the tie band"
            kth_misses += len(diff) // 2
        gs = g["topk_score"][j][: valid.size]
        exp = s["scores64"][[pos_of[int(x)] for x in valid]]
        assert np.all(np.abs(gs - exp) <= SCORE_ATOL), f"row {j}: selected score mismatch"
        gidx_rows.append(gi)
    # ---- S5 sparse MLA on the GPU's own selection
    ref_o, ref_l = opl.sparse_mla_rows(rows, gidx_rows, inp["q"], wl.act_fmt, kv_data,
                                       wl.kv_fmt, kv_scale, wl.scale, wl.d_latent)
    abs_gate, rel_gate = _mla_gate(wl)
    for key_o, key_l in (("out", "lse"), ("out_prefill_kernel", "lse_prefill_kernel")):
        if key_o not in g:
            continue
        got_o = g[key_o][rows]
        err = np.abs(got_o - ref_o).max()
        rel = err / np.abs(ref_o).max()
        lerr = np.abs(g[key_l][rows] - ref_l).max()
        gp.say(f"  {wl.name} {key_o}: max|dO|={err:.3e} rel={rel:.3e} max|dlse|={lerr:.3e}"
               f" top-k swaps within band={kth_misses}")
        assert err <= abs_gate and rel <= rel_gate, (err, rel)
        assert lerr <= 1e-3, lerr


PREFILL_SMALL = ["tiny_prefill_t256_cp4", "tiny_prefill_dense", "tiny_prefill_bf16",
                 "small_prefill_3req_cp4", "small_prefill_3req_cp4_fp8",
                 "small_prefill_topk2048", "small_prefill_sharp", "small_prefill_topk777",
                 "small_prefill_cp1", "small_prefill_cp16"]
PREFILL_FULL = ["prefill_t8000_cp8", "prefill_6req_t25305_cp8", "prefill_t65536_cp8_fp8"]


def _check_prefill(name, all_rows):
    wl = get(name)
    T, cp, r = wl.num_tokens, wl.cp_size, wl.cp_rank
    n = orr.local_count(T, cp, r)
    inp = draw_prefill(wl, n)
    g = gp.run_prefill(wl, inp)
    om = orr.split_metadata(inp["cu_seqlens"], cp, r)
    # S1: metadata and the row gather, bit-exact
    for key in ("global_idx", "batch_idx", "local_cu", "kv_start", "kv_len"):
        assert np.array_equal(g[key], om[key]), key
    assert np.array_equal(g["rows"], orr.split_rows(inp["input_ids"], cp, r))
    # all-gather stand-in built by the split kernel == the oracle's rank concat
    kv_bytes = np.ascontiguousarray(inp["kv"]).view(np.uint8).reshape(T, -1)
    cat = orr.rank_concat(kv_bytes, cp, g["slot"], pad_value=0xFF)
    assert np.array_equal(g["kv_cat_bytes"].reshape(cat.shape), cat)
    # S2: rerange restores logical order, bit-exact
    assert np.array_equal(g["kv_bytes"].reshape(T, -1), orr.rerange(cat, T, cp, g["slot"]))
    assert np.array_equal(g["kv_bytes"].reshape(T, -1), kv_bytes)
    ki_bytes = np.ascontiguousarray(inp["k_idx"]).view(np.uint8).reshape(T, -1)
    assert np.array_equal(g["ki_bytes"].reshape(T, -1), ki_bytes)
    # S3 on every row (a property that holds at any size): each query's
    # scores over its whole causal range were written, and nothing past it
    sc = g["scores"]
    written = np.arange(sc.shape[1])[None, :] < g["kv_len"].astype(np.int64)[:, None]
    assert np.isfinite(sc[written]).all(), "a causal score was not written"
    assert np.isnan(sc[~written]).all(), "a score past kv_len was written"
    del written
    rows = list(range(n)) if all_rows else _sample_rows(n, wl.seed, om["local_cu"])
    if not all_rows:   # every request's first and last local row is among them
        for lo, hi in zip(om["local_cu"][:-1], om["local_cu"][1:]):
            assert hi == lo or (lo in rows and hi - 1 in rows)
    gp.say(f"  oracle on {len(rows)} of {n} rows")
    sel = opl.indexer_topk_rows(rows, om, inp["q_idx"], wl.act_fmt, inp["w"], inp["k_idx"],
                                wl.kv_fmt, inp["k_idx_scale"], wl.topk)
    _check_rows(wl, g, sel, rows, inp, inp["kv"], inp["kv_scale"])


@pytest.mark.parametrize("name", PREFILL_SMALL)
def test_prefill_small_all_rows(name):
    _check_prefill(name, all_rows=True)


@pytest.mark.parametrize("name", PREFILL_FULL)
def test_prefill_full_size_sampled_rows(name):
    _check_prefill(name, all_rows=False)


def _check_decode(name, all_rows):
    wl = get(name)
    inp = draw_decode(wl)
    g = gp.run_decode(wl, inp)
    meta = opl.decode_metadata(inp["lengths"])
    rows = list(range(wl.n_req)) if all_rows else _sample_rows(wl.n_req, wl.seed)
    sel = opl.indexer_topk_rows(rows, meta, inp["q_idx"], wl.act_fmt, inp["w"], inp["k_idx"],
                                wl.kv_fmt, inp["k_idx_scale"], wl.topk,
                                page_table=inp["page_table"], page_size=wl.page_size)
    _check_rows(wl, g, sel, rows, inp, inp["kv"], inp["kv_scale"])


def test_decode_small_all_rows():
    _check_decode("small_decode_paged", all_rows=True)


def test_decode_small_fp8_all_rows():
    _check_decode("small_decode_paged_fp8", all_rows=True)


def test_decode_small_fp8_topk_off_the_tile_grid():
    _check_decode("small_decode_topk333_fp8", all_rows=True)


@pytest.mark.parametrize("name", ["small_decode_splits", "small_decode_splits_fp8"])
def test_decode_split_partials_with_empty_splits(name):
    _check_decode(name, all_rows=True)


def test_decode_full_size_all_requests():
    _check_decode("decode_32req_paged", all_rows=True)


def test_decode_contexts_past_65536_keys():
    # rows longer than the one-pass selection takes: top-k in two phases
    # (segments, then their candidates)
    _check_decode("long_decode_paged", all_rows=True)


# ------------------------------------------------------------------ edges

def test_ranks_without_tokens_and_empty_requests():
    cu = torch.tensor([0, 3, 3, 5], dtype=torch.int32, device=gp.DEV)
    for r in range(8):
        meta = ds.cp_split_metadata(cu, 5, 8, r)
        om = orr.split_metadata([0, 3, 3, 5], 8, r)
        torch.cuda.synchronize()
        for key in ("global_idx", "batch_idx", "local_cu", "kv_start", "kv_len"):
            assert np.array_equal(meta[key].cpu().numpy(), om[key]), (r, key)


@pytest.mark.parametrize("row_shape,dtype", [((3,), torch.uint8), ((1,), torch.int32),
                                             ((2,), torch.int32), ((80,), torch.float32),
                                             ((576,), torch.uint8), ((128,), torch.bfloat16)])
def test_rerange_host_built_concat_all_row_sizes(row_shape, dtype):
    elem = torch.empty((), dtype=dtype).element_size()
    rb = int(np.prod(row_shape)) * elem
    for T, cp in ((1, 4), (13, 4), (1001, 8), (4096, 3)):
        x = np.random.default_rng(T + 1).integers(0, 256, size=(T, rb), dtype=np.uint8)
        slot = orr.local_count(T, cp, 0)
        cat = orr.rank_concat(x, cp, slot, pad_value=0xFF)
        src = torch.from_numpy(cat).to(gp.DEV).view(dtype).reshape((cp * slot,) + row_shape)
        got = ds.kv_rerange(src, slot, T, cp)
        torch.cuda.synchronize()
        assert np.array_equal(gp.raw_bytes(got).reshape(T, rb), orr.rerange(cat, T, cp, slot))


def test_mla_rejects_scale_that_is_not_positive_and_finite():
    # the softmax maximum is taken on raw dot products and scaled afterwards,
    # which needs sm_scale > 0; the host check returns DS_ERR_INVALID_ARG
    # before any launch, and the output is left untouched
    q = torch.zeros(2, 128, 576, device=gp.DEV, dtype=torch.bfloat16)
    kv = torch.zeros(40, 576, device=gp.DEV, dtype=torch.bfloat16)
    idx = torch.arange(64, device=gp.DEV, dtype=torch.int32).view(2, 32) % 40
    for fn in (ds.sparse_mla_prefill, ds.sparse_mla_decode):
        for sc in (0.0, -0.5, float("inf"), float("nan")):
            out = torch.full((2, 128, 512), 7.0, device=gp.DEV, dtype=torch.bfloat16)
            with pytest.raises(ds.DS32CPError) as ei:
                fn(q, kv, idx, sc, 512, out=out)
            assert ei.value.status == 1, ei.value   # DS_ERR_INVALID_ARG
            torch.cuda.synchronize()
            assert bool((out == 7.0).all())
    o, _ = ds.sparse_mla_prefill(q, kv, idx, 1e-3, 512)   # a valid scale still runs
    torch.cuda.synchronize()
    assert bool((o == 0).all())


def test_mla_empty_and_out_of_range_rows():
    wl = get("tiny_prefill_bf16")
    rng = np.random.default_rng(5)
    q = torch.randn(3, 128, 576, device=gp.DEV).bfloat16() / 24
    kv = torch.randn(50, 576, device=gp.DEV).bfloat16() / 24
    idx = torch.full((3, 64), -1, dtype=torch.int32, device=gp.DEV)
    idx[1, :5] = torch.tensor([3, 7, 50, 1000, 9], dtype=torch.int32)   # 50, 1000 out of range
    idx[2, 10:20] = torch.from_numpy(rng.permutation(50)[:10].astype(np.int32)).to(gp.DEV)
    out, lse = ds.sparse_mla_prefill(q, kv, idx, wl.scale, 512)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isinf(lse[0])) and torch.all(lse[0] < 0)
    qn = q.view(torch.int16).cpu().numpy().view(np.uint16)
    kvn = kv.view(torch.int16).cpu().numpy().view(np.uint16)
    for j, sel in ((1, [3, 7, 9]), (2, idx[2, 10:20].cpu().tolist())):
        ro, rl = opl.sparse_mla_rows([j], [np.array(sel)], qn, "bf16", kvn, "bf16", None,
                                     wl.scale, 512)
        err = np.abs(out[j].float().cpu().numpy() - ro[0]).max()
        assert err <= 1e-2 * np.abs(ro[0]).max(), err
        assert np.abs(lse[j].cpu().numpy() - rl[0]).max() <= 1e-3


def test_decode_page_boundaries():
    # lengths 1, 63, 64, 65, 129 exercise partial and exact pages
    lengths = np.array([1, 63, 64, 65, 129], dtype=np.int32)
    ps = 64
    pages = [-(-int(L) // ps) for L in lengths]
    rng = np.random.default_rng(9)
    perm = rng.permutation(sum(pages)).astype(np.int32)
    table = np.full((5, max(pages)), -1, dtype=np.int32)
    off = 0
    for i, k in enumerate(pages):
        table[i, :k] = perm[off: off + k]
        off += k
    rows = sum(pages) * ps
    ki = (rng.standard_normal((rows, 128)) / np.sqrt(128)).astype(np.float32)
    qi = (rng.standard_normal((5, 64, 128)) / np.sqrt(128)).astype(np.float32)
    w = (rng.standard_normal((5, 64)) / 8).astype(np.float32)
    from synth.draw import to_bf16_bits
    ki_b, qi_b = to_bf16_bits(ki), to_bf16_bits(qi)
    meta = ds.decode_metadata(torch.from_numpy(lengths).to(gp.DEV))
    idx, _ = ds.indexer_topk(gp.to_dev(qi_b, "bf16"), torch.from_numpy(w).to(gp.DEV),
                             gp.to_dev(ki_b, "bf16"), meta["kv_start"], meta["kv_len"],
                             int(lengths.max()), 16, q_req=meta["q_req"],
                             page_table=torch.from_numpy(table).to(gp.DEV), page_size=ps)
    torch.cuda.synchronize()
    om = opl.decode_metadata(lengths)
    sel = opl.indexer_topk_rows(range(5), om, qi_b, "bf16", w, ki_b, "bf16", None, 16,
                                page_table=table, page_size=ps)
    gi = idx.cpu().numpy()
    for j, s in enumerate(sel):
        assert set(gi[j][gi[j] >= 0].tolist()) == set(s["topk_idx"][s["topk_idx"] >= 0].tolist())


@pytest.mark.parametrize("kfmt", ["bf16", "fp8"])
def test_prefill_indexer_arbitrary_ranges_and_two_launches(kfmt):
    # The contiguous (prefill) indexer on ranges no causal prefill has:
    # empty ranges, starts inside a 64-key half and on either side of a
    # 2048-key score window, ranges ending at the last key row, and 8200
    # queries, so that the query blocks (8 queries each) take two launches.
    # Every row: scores written over exactly its range.  Sampled rows (the
    # blocks around the launch boundary and every planted case) against the
    # oracle.
    rng = np.random.default_rng(31 if kfmt == "bf16" else 32)
    K, n, max_len = 5000, 8200, 3000
    kv_start = rng.integers(0, K, n).astype(np.int32)
    kv_len = np.minimum(rng.integers(0, max_len + 1, n), K - kv_start).astype(np.int32)
    planted = {0: (0, 0), 5: (0, 1), 6: (63, 2), 7: (2047, 2), 8: (2048, 700), 9: (2040, 2100),
               100: (4999, 1), 101: (K - 3000, 3000), 8183: (1, 0), 8184: (4095, 905),
               8191: (0, 3000), 8192: (130, 2), 8199: (4000, 1000)}
    for j, (st, ln) in planted.items():
        kv_start[j], kv_len[j] = st, ln
    kv_len[1000:1040] = 0                        # five query blocks with no work at all
    from synth.draw import to_bf16_bits, to_e4m3fn_blocks
    ki = (rng.standard_normal((K, 128)) / np.sqrt(128)).astype(np.float32)
    ki_v, ki_scale = (to_bf16_bits(ki), None) if kfmt == "bf16" else to_e4m3fn_blocks(ki)
    qi_b = to_bf16_bits((rng.standard_normal((n, 64, 128)) / np.sqrt(128)).astype(np.float32))
    w = (rng.standard_normal((n, 64)) / 8).astype(np.float32)
    ks_dev = None if ki_scale is None else torch.from_numpy(ki_scale).to(gp.DEV)
    gp.say(f"[gpu] prefill indexer, arbitrary ranges, {n} queries, {kfmt} keys")
    sc = ds.indexer_scores(gp.to_dev(qi_b, "bf16"), torch.from_numpy(w).to(gp.DEV),
                           gp.to_dev(ki_v, kfmt), torch.from_numpy(kv_start).to(gp.DEV),
                           torch.from_numpy(kv_len).to(gp.DEV), max_len, k_scale=ks_dev)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    written = np.arange(max_len)[None, :] < kv_len.astype(np.int64)[:, None]
    assert np.isfinite(sc[written]).all(), "a score in range was not written"
    assert np.isnan(sc[~written]).all(), "a score past the range was written"
    rows = sorted(set(planted) | set(range(8176, 8200)) | set(range(1000, 1041, 8)) |
                  set(rng.choice(n, 24, replace=False).tolist()))
    meta = {"kv_start": kv_start, "kv_len": kv_len}
    sel = opl.indexer_topk_rows(rows, meta, qi_b, "bf16", w, ki_v, kfmt, ki_scale, 16)
    for j, s in zip(rows, sel):
        L = int(kv_len[j])
        assert np.all(np.abs(sc[j, :L] - s["scores64"]) <= SCORE_ATOL), f"row {j}: score error"


@pytest.mark.parametrize("kfmt", ["bf16", "fp8"])
@pytest.mark.parametrize("ps", [1, 16, 48, 64])
def test_decode_indexer_page_sizes_and_offsets(ps, kfmt):
    # Paged indexer scores and top-k with page sizes that do and do not
    # divide the 32-position work unit, queries whose causal range starts
    # inside the request (kv_start > 0), and lengths around unit edges.
    lengths = np.array([1, 31, 32, 33, 700, 2500], dtype=np.int32)
    kv_start = np.array([0, 3, 0, 40, 17, 0], dtype=np.int32)
    span = lengths + kv_start
    pages = [-(-int(x) // ps) for x in span]
    rng = np.random.default_rng(100 + ps)
    perm = rng.permutation(sum(pages)).astype(np.int32)
    table = np.full((lengths.size, max(pages)), -1, dtype=np.int32)
    off = 0
    for i, k in enumerate(pages):
        table[i, :k] = perm[off: off + k]
        off += k
    rows = sum(pages) * ps
    from synth.draw import to_bf16_bits, to_e4m3fn_blocks
    ki = (rng.standard_normal((rows, 128)) / np.sqrt(128)).astype(np.float32)
    ki_v, ki_scale = (to_bf16_bits(ki), None) if kfmt == "bf16" else to_e4m3fn_blocks(ki)
    qi_b = to_bf16_bits((rng.standard_normal((lengths.size, 64, 128)) / np.sqrt(128)).astype(np.float32))
    w = (rng.standard_normal((lengths.size, 64)) / 8).astype(np.float32)
    meta = {"q_req": np.arange(lengths.size, dtype=np.int32), "kv_start": kv_start, "kv_len": lengths}
    dev = {k: torch.from_numpy(v).to(gp.DEV) for k, v in meta.items()}
    ks_dev = None if ki_scale is None else torch.from_numpy(ki_scale).to(gp.DEV)
    args = (gp.to_dev(qi_b, "bf16"), torch.from_numpy(w).to(gp.DEV), gp.to_dev(ki_v, kfmt),
            dev["kv_start"], dev["kv_len"], int(lengths.max()))
    paging = dict(q_req=dev["q_req"], page_table=torch.from_numpy(table).to(gp.DEV), page_size=ps)
    sc = ds.indexer_scores(*args, k_scale=ks_dev, **paging)
    idx, _ = ds.indexer_topk(*args, 16, k_scale=ks_dev, **paging)
    torch.cuda.synchronize()
    sc, gi = sc.cpu().numpy(), idx.cpu().numpy()
    sel = opl.indexer_topk_rows(range(lengths.size), meta, qi_b, "bf16", w, ki_v, kfmt, ki_scale, 16,
                                page_table=table, page_size=ps)
    for j, s in enumerate(sel):
        L = int(lengths[j])
        assert np.all(np.abs(sc[j, :L] - s["scores64"]) <= SCORE_ATOL), f"row {j}: score error"
        got = set(gi[j][gi[j] >= 0].tolist())
        exp = set(s["topk_idx"][s["topk_idx"] >= 0].tolist())
        if L <= 16:
            assert got == exp, f"row {j}: must select every causal key"
        else:
            pos_of = {int(x): p for p, x in enumerate(s["key_rows"].tolist())}
            kth = s["scores64"][s["sel_pos"][-1]]
            far = [x for x in got ^ exp if abs(s["scores64"][pos_of[x]] - kth) > TOPK_BAND]
            assert not far, f"row {j}: selections outside the tie band"


def test_integer_outputs_repeatable():
    wl = get("small_prefill_3req_cp4")
    n = orr.local_count(wl.num_tokens, wl.cp_size, wl.cp_rank)
    inp = draw_prefill(wl, n)
    a = gp.run_prefill(wl, inp, want_scores=False)
    b = gp.run_prefill(wl, inp, want_scores=False)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


@pytest.mark.parametrize("name", ["small_decode_paged", "small_decode_splits_fp8"])
def test_decode_outputs_repeatable(name):
    # split partials merged by the combine kernel, fp8 and bf16 pools: the
    # same inputs give the same selection and bit-identical outputs
    wl = get(name)
    inp = draw_decode(wl)
    a = gp.run_decode(wl, inp, want_scores=False)
    b = gp.run_decode(wl, inp, want_scores=False)
    for key in ("topk_idx", "topk_score", "out", "lse"):
        assert np.array_equal(a[key].view(np.uint32) if a[key].dtype == np.float32 else a[key],
                              b[key].view(np.uint32) if b[key].dtype == np.float32 else b[key]), key


@pytest.mark.parametrize("heads", [32, 64])
def test_mla_head_counts_below_128(heads):
    # the ABI takes any head count that is a multiple of 32 (up to 128): the
    # kernels for 32 and 64 heads (one or two waves per query), prefill and
    # decode (split partials merged by the combine), against the oracle
    rng = np.random.default_rng(40 + heads)
    g = torch.Generator(device="cpu").manual_seed(40 + heads)
    n, rows, k = 20, 2000, 256
    q = (torch.randn(n, heads, 576, generator=g) / 24).bfloat16().to(gp.DEV)
    kv = (torch.randn(rows, 576, generator=g) / 24).bfloat16().to(gp.DEV)
    idx = np.full((n, k), -1, dtype=np.int32)
    for j in range(n):
        cnt = int(rng.integers(1, k + 1)) if j % 3 else k   # ragged tails
        idx[j, :cnt] = rng.choice(rows, cnt, replace=False)
    idx_t = torch.from_numpy(idx).to(gp.DEV)
    scale = 1.0 / 24.0
    qb, kvb = q.view(torch.int16).cpu().numpy(), kv.view(torch.int16).cpu().numpy()
    ref_o, ref_l = opl.sparse_mla_rows(list(range(n)), list(idx), qb, "bf16", kvb, "bf16", None,
                                       scale, 512)
    for fn in (ds.sparse_mla_prefill, ds.sparse_mla_decode):
        o, lse = fn(q, kv, idx_t, scale, 512)
        torch.cuda.synchronize()
        err = np.abs(o.float().cpu().numpy() - ref_o).max()
        rel = err / np.abs(ref_o).max()
        lerr = np.abs(lse.cpu().numpy() - ref_l).max()
        gp.say(f"  {heads} heads {fn.__name__}: max|dO|={err:.3e} rel={rel:.3e} max|dlse|={lerr:.3e}")
        assert err <= 2e-2 and rel <= 1e-2, (fn.__name__, err, rel)
        assert lerr <= 1e-3, (fn.__name__, lerr)
    # decode with few queries and more rows per query: four splits each
    q4 = q[:4].contiguous()
    idx4 = np.full((4, 1024), -1, dtype=np.int32)
    for j in range(4):
        idx4[j, : 1024 - 100 * j] = rng.choice(rows, 1024 - 100 * j, replace=False)
    o4, l4 = ds.sparse_mla_decode(q4, kv, torch.from_numpy(idx4).to(gp.DEV), scale, 512)
    torch.cuda.synchronize()
    r4o, r4l = opl.sparse_mla_rows(list(range(4)), list(idx4), qb, "bf16", kvb, "bf16", None,
                                   scale, 512)
    err = np.abs(o4.float().cpu().numpy() - r4o).max()
    assert err <= 2e-2 and err / np.abs(r4o).max() <= 1e-2, err
    assert np.abs(l4.cpu().numpy() - r4l).max() <= 1e-3


def test_topk_ties_in_the_threshold_bin_and_length_limits():
    # rows whose k-th largest score is shared by several keys while the
    # threshold's 12-bit bin stays small (the lowest tied positions are
    # taken), rows whose tied keys are all taken, rows at 65536 keys and one
    # past it, an odd length, and a row that starts at an odd float offset;
    # selected scores are returned too.  The decision is on the same float32
    # values: the selected sets and scores must equal the oracle's exactly.
    rng = np.random.default_rng(77)
    k = 2048
    Lmax = 65537
    specs = []
    base = rng.standard_normal(40000).astype(np.float32)
    order = np.argsort(-base, kind="stable")
    r0 = base.copy()
    r0[order[2000:2060]] = base[order[2030]]        # 60 ties straddle rank k: 48 taken
    specs.append(r0)
    r1 = base.copy()
    r1[order[2040:2048]] = base[order[2047]]        # 8 ties, all taken
    specs.append(r1)
    r2 = base.copy()
    r2[order[2048:2100]] = base[order[2047]]        # the k-th key and 52 equal ones below it
    specs.append(r2)
    specs.append(rng.standard_normal(65536).astype(np.float32) * 3.0 - 1.0)
    specs.append(rng.standard_normal(65537).astype(np.float32))
    specs.append(rng.standard_normal(40001).astype(np.float32))
    r6 = -np.abs(rng.standard_normal(30000)).astype(np.float32)   # all negative, with -0.0 and +0.0
    r6[:10] = -0.0
    r6[10:20] = 0.0
    specs.append(r6)
    lens = np.array([x.size for x in specs], dtype=np.int32)
    stride = Lmax + 2                                # rows start at 4-byte (not 16-byte) offsets
    scores = np.full((len(specs), stride), np.nan, dtype=np.float32)
    for i, r in enumerate(specs):
        scores[i, : lens[i]] = r
    dev_scores = torch.from_numpy(scores).to(gp.DEV)
    kv_start = torch.zeros(len(specs), dtype=torch.int32, device=gp.DEV)
    kv_len = torch.from_numpy(lens).to(gp.DEV)
    idx, sc = ds.topk_select(dev_scores, kv_start, kv_len, Lmax, k, Lmax, want_score=True)
    torch.cuda.synchronize()
    got, got_sc = idx.cpu().numpy(), sc.cpu().numpy()
    for i in range(len(specs)):
        row = scores[i, : lens[i]]
        want = np.sort(sa.topk_positions(row, k))
        assert np.array_equal(got[i], want), f"row {i}: {np.setxor1d(got[i], want).size} differences"
        want_sc = row[want] + np.float32(0.0)       # -0.0 is reported as +0.0
        assert np.array_equal(got_sc[i], want_sc), f"row {i}: scores differ"


def test_topk_many_long_rows_three_workgroups_per_cu():
    # A launch of more than 512 rows longer than 16384 keys takes the
    # 512-thread selection that runs three rows per CU and reads each row
    # twice from memory instead of caching it in LDS (its general path
    # stages blocks of 4096 keys).  The planted rows of the two tests around
    # this one, at a stride that starts every row at a 4-byte offset, among
    # random rows of 2049 to 65536 keys; sets and returned scores must equal
    # the oracle's exactly.
    rng = np.random.default_rng(91)
    k, Lmax, n = 2048, 65536, 530
    base = rng.standard_normal(40000).astype(np.float32)
    order = np.argsort(-base, kind="stable")
    specs = []
    for lo, hi, src in ((2000, 2060, 2030), (2040, 2048, 2047), (2048, 2100, 2047)):
        r = base.copy()
        r[order[lo:hi]] = base[order[src]]
        specs.append(r)
    specs.append(rng.standard_normal(65536).astype(np.float32) * 3.0 - 1.0)
    specs.append(rng.standard_normal(40001).astype(np.float32))
    r = -np.abs(rng.standard_normal(30000)).astype(np.float32)
    r[:10], r[10:20] = -0.0, 0.0
    specs.append(r)
    specs.append(np.full(40000, 0.5, dtype=np.float32))                       # all tied
    specs.append(rng.choice(np.array([-1.0, 0.25, 0.5, 2.0], dtype=np.float32), 40000))
    r = (1.0 + rng.random(36000)).astype(np.float32)
    r[rng.choice(36000, 2000, replace=False)] = 4.0
    specs.append(r)
    r = rng.standard_normal(40000).astype(np.float32)
    r[(np.arange(2048) * 40000 + 20000) // 2048] = -5.0
    specs.append(r)
    specs.append(np.concatenate([rng.standard_normal(30000).astype(np.float32) * 1e-3 + 7.0,
                                 np.zeros(10000, np.float32)]))
    specs += [rng.standard_normal(m).astype(np.float32) for m in (1000, 2048, 2049, 16385)]
    while len(specs) < n:
        specs.append(rng.standard_normal(int(rng.integers(2049, Lmax + 1))).astype(np.float32))
    lens = np.array([x.size for x in specs], dtype=np.int32)
    stride = Lmax + 1
    scores = np.full((n, stride), np.nan, dtype=np.float32)
    for i, r in enumerate(specs):
        scores[i, : lens[i]] = r
    gp.say(f"[gpu] top-k of {n} rows up to {Lmax} keys (three rows per CU)")
    dev_scores = torch.from_numpy(scores).to(gp.DEV)
    kv_start = torch.zeros(n, dtype=torch.int32, device=gp.DEV)
    kv_len = torch.from_numpy(lens).to(gp.DEV)
    idx, sc = ds.topk_select(dev_scores, kv_start, kv_len, Lmax, k, Lmax, want_score=True)
    torch.cuda.synchronize()
    got, got_sc = idx.cpu().numpy(), sc.cpu().numpy()
    for i in range(n):
        row = scores[i, : lens[i]]
        want = np.sort(sa.topk_positions(row, k))
        if want.size < k:
            want = np.concatenate([want, np.full(k - want.size, -1)])
        assert np.array_equal(got[i], want), f"row {i}: {np.setxor1d(got[i], want).size} differences"
        m = min(k, int(lens[i]))
        want_sc = row[want[:m]] + np.float32(0.0)  # -0.0 is reported as +0.0
        assert np.array_equal(got_sc[i][:m], want_sc), f"row {i}: scores differ"


def test_topk_rows_longer_than_the_cache():
    # rows longer than the 32768-key LDS cache: the threshold bucket is
    # compacted into the cache after the first radix pass when it fits, and
    # the row is re-read per pass when it does not; ties go to the lower
    # position.  The decision is on the same float32 values, so the selected
    # sets must equal the oracle's exactly.
    rng = np.random.default_rng(51)
    L, k = 40000, 2048
    rows = []
    rows.append(rng.standard_normal(L).astype(np.float32))                 # compacted bucket
    rows.append(np.full(L, 0.5, dtype=np.float32))                         # bucket > cache: all tied
    rows.append(rng.choice(np.array([-1.0, 0.25, 0.5, 2.0], dtype=np.float32), L))   # heavy ties
    r3 = (1.0 + rng.random(L)).astype(np.float32)                          # 38000 in [1, 2) ...
    r3[rng.choice(L, 2000, replace=False)] = 4.0                           # ... 2000 above: bucket > cache
    rows.append(r3)
    rows.append(rng.standard_normal(L).astype(np.float32))                 # short row (select all)
    # every 20th position low (a strided pattern), and a clustered row
    r5 = rng.standard_normal(L).astype(np.float32)
    r5[(np.arange(2048) * L + L // 2) // 2048] = -5.0
    rows.append(r5)
    r6 = rng.standard_normal(30000).astype(np.float32) * 1e-3 + 7.0       # clustered, in the cache
    rows.append(np.concatenate([r6, np.zeros(L - 30000, np.float32)]))
    lens = np.array([L, L, L, 36000, 1000, L, 30000], dtype=np.int32)
    scores = np.full((len(rows), L), np.nan, dtype=np.float32)
    for i, r in enumerate(rows):
        scores[i, : lens[i]] = r[: lens[i]]
    dev_scores = torch.from_numpy(scores).to(gp.DEV)
    kv_start = torch.zeros(len(rows), dtype=torch.int32, device=gp.DEV)
    kv_len = torch.from_numpy(lens).to(gp.DEV)
    idx, _ = ds.topk_select(dev_scores, kv_start, kv_len, L, k, L)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for i in range(len(rows)):
        want = np.sort(sa.topk_positions(scores[i, : lens[i]], k))
        g_i = got[i][got[i] >= 0]
        assert (np.diff(g_i) > 0).all(), f"row {i}: not in position order"
        assert np.array_equal(g_i, want), f"row {i}: {np.setxor1d(g_i, want).size} differences"
        assert (got[i][g_i.size:] == -1).all()
