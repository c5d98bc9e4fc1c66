"""Pins of the indexer / top-k / sparse-MLA oracle.

Each test ties the oracle to something other than itself: library routines
on special cases (torch's dtype conversions, torch's
scaled_dot_product_attention when top-k covers the whole causal context,
scipy's logsumexp), closed forms (relu(x) - relu(-x) = x, one-key and
zero-query attention), hand-worked numbers, brute-force characterisation
of the top-k set, and invariances (linearity in the head weights,
order of selected rows, context-parallel invariance end to end).
"""

import itertools

import numpy as np
import pytest
import scipy.special
import torch

from oracle import pipeline as pl
from oracle import round_robin_cp as rr
from oracle import sparse_attention as sa


# ---------------------------------------------------------------- formats

def test_bf16_decode_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = sa.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = sa.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                       # S.1111.111 for both signs
    assert np.array_equal(got[~nan], ref[~nan])
    # hand values: 1.0 = 0.0111.000, 448 = 0.1111.110, smallest subnormal
    # 2^-9 = 0.0000.001, smallest normal 2^-6 = 0.0001.000
    assert got[0x38] == 1.0 and got[0xB8] == -1.0
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_fp8_block_scale_is_per_128_rows():
    codes = np.full((300, 2), 0x38, dtype=np.uint8)        # every value 1.0
    scale = np.array([2.0, 3.0, 5.0], dtype=np.float32)
    vals = sa.decode_rows(codes, "fp8", scale, np.arange(300))
    assert (vals[:128] == 2.0).all() and (vals[128:256] == 3.0).all()
    assert (vals[256:] == 5.0).all()
    assert sa.decode_rows(codes, "fp8", scale, [127, 128])[:, 0].tolist() == [2.0, 3.0]


# ---------------------------------------------------------------- indexer

def test_indexer_hand_example():
    # two heads, two dims; keys k0 = (1, 1), k1 = (2, -3), k2 = (0, 0)
    q = np.array([[1.0, 2.0], [3.0, -1.0]])
    keys = np.array([[1.0, 1.0], [2.0, -3.0], [0.0, 0.0]])
    # w = (0.5, 2):  k0: 0.5*relu(3) + 2*relu(2) = 5.5
    #                k1: 0.5*relu(-4) + 2*relu(9) = 18
    #                k2: 0
    assert sa.indexer_scores_row(q, np.array([0.5, 2.0]), keys).tolist() == [5.5, 18.0, 0.0]
    # negative weight: w = (-1, 1): k0: -3 + 2 = -1, k1: 0 + 9 = 9
    assert sa.indexer_scores_row(q, np.array([-1.0, 1.0]), keys).tolist() == [-1.0, 9.0, 0.0]


def test_indexer_relu_identity_closed_form():
    # relu(x) - relu(-x) = x, so I(q, k) - I(q, -k) = (w @ q) . k
    rng = np.random.default_rng(1)
    q = rng.standard_normal((8, 16))
    w = rng.standard_normal(8)
    keys = rng.standard_normal((40, 16))
    diff = sa.indexer_scores_row(q, w, keys) - sa.indexer_scores_row(q, w, -keys)
    assert np.allclose(diff, keys @ (w @ q), rtol=0, atol=1e-12)


def test_indexer_linear_in_weights_and_head_permutation():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 8))
    keys = rng.standard_normal((25, 8))
    w1, w2 = rng.standard_normal(6), rng.standard_normal(6)
    s = lambda w: sa.indexer_scores_row(q, w, keys)  # noqa: E731
    assert np.allclose(s(w1 + 2.5 * w2), s(w1) + 2.5 * s(w2), atol=1e-12)
    perm = rng.permutation(6)
    assert np.allclose(sa.indexer_scores_row(q[perm], w1[perm], keys), s(w1), atol=1e-12)


def test_indexer_key_locality():
    rng = np.random.default_rng(3)
    q, w = rng.standard_normal((4, 8)), rng.standard_normal(4)
    keys = rng.standard_normal((12, 8))
    base = sa.indexer_scores_row(q, w, keys)
    keys2 = keys.copy()
    keys2[7] = rng.standard_normal(8)
    changed = sa.indexer_scores_row(q, w, keys2) != base
    assert changed.tolist() == [p == 7 for p in range(12)]


def test_paged_key_rows_hand_example():
    table = np.array([[2, 0, -1]], dtype=np.int32)
    assert sa.paged_key_rows(table, 4, 0, 0, 6).tolist() == [8, 9, 10, 11, 0, 1]
    ident = np.array([[0, 1, 2]], dtype=np.int32)
    assert sa.paged_key_rows(ident, 4, 0, 0, 11).tolist() == list(range(11))


# ---------------------------------------------------------------- top-k

def _is_topk(scores, sel, k):
    """Characterisation: sel holds min(k, L) distinct positions, and every
    selected (score, -pos) beats every unselected one."""
    L = len(scores)
    if len(sel) != min(k, L) or len(set(sel)) != len(sel):
        return False
    rest = [p for p in range(L) if p not in set(sel)]
    key = lambda p: (scores[p], -p)  # noqa: E731
    return all(key(a) > key(b) for a in sel for b in rest)


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 9))
    scores = rng.integers(-1, 3, size=L).astype(np.float32)   # many ties
    for k in range(1, L + 2):
        sel = sa.topk_positions(scores, k).tolist()
        assert _is_topk(scores.tolist(), sel, k)
        # brute force: the lexicographically best k-subset
        best = max(itertools.combinations(range(L), min(k, L)),
                   key=lambda c: sorted(((scores[p], -p) for p in c), reverse=True))
        assert sorted(sel) == sorted(best)


def test_topk_partition_second_implementation():
    rng = np.random.default_rng(7)
    for _ in range(50):
        L = int(rng.integers(1, 400))
        k = int(rng.integers(1, 300))
        scores = np.round(rng.standard_normal(L), 1).astype(np.float32)
        sel = set(sa.topk_positions(scores, k).tolist())
        if k >= L:
            assert sel == set(range(L))
            continue
        kth = np.partition(scores, L - k)[L - k]             # k-th largest value
        above = set(np.flatnonzero(scores > kth).tolist())
        ties = np.flatnonzero(scores == kth)[: k - len(above)]
        assert sel == above | set(ties.tolist())


def test_topk_order_and_signed_zero():
    s = np.array([0.0, -0.0, 1.0, 0.0], dtype=np.float32)
    # -0.0 and +0.0 are equal scores: ties go to the lower position
    assert sa.topk_positions(s, 3).tolist() == [2, 0, 1]
    assert sa.pad_indices(np.array([4, 2]), 4).tolist() == [4, 2, -1, -1]


# ---------------------------------------------------------------- sparse MLA

def _dense_causal_sdpa(q, kv, d_latent, scale):
    """torch's SDPA (float64) with an explicit causal boolean mask: query at
    position p sees keys 0..p.  q [T, H, D], kv [T, D]."""
    T, H, _ = q.shape
    qt = torch.from_numpy(q).permute(1, 0, 2)                  # [H, T, D]
    kt = torch.from_numpy(kv).unsqueeze(0).expand(H, T, -1)   # shared row
    vt = torch.from_numpy(np.ascontiguousarray(kv[:, :d_latent])).unsqueeze(0).expand(H, T, -1)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("scale", [80 ** -0.5, 80 ** 0.5])
def test_mla_topk_covering_context_is_dense_causal_attention(scale):
    rng = np.random.default_rng(11)
    T, H, Dl, Dr = 37, 4, 64, 16
    q = rng.standard_normal((T, H, Dl + Dr)) / np.sqrt(Dl + Dr)
    kv = rng.standard_normal((T, Dl + Dr)) / np.sqrt(Dl + Dr)
    ref = _dense_causal_sdpa(q, kv, Dl, scale)
    for p in range(T):
        out, _ = sa.sparse_mla_row(q[p], kv[np.arange(p + 1)], scale, Dl)
        assert np.allclose(out, ref[p], rtol=0, atol=1e-12)


def test_mla_one_key_and_zero_query_closed_forms():
    rng = np.random.default_rng(12)
    H, D, Dl = 3, 10, 8
    q = rng.standard_normal((H, D))
    keys = rng.standard_normal((5, D))
    out, lse = sa.sparse_mla_row(q, keys[:1], 0.7, Dl)
    assert np.allclose(out, np.broadcast_to(keys[0, :Dl], (H, Dl)), atol=1e-15)
    assert np.allclose(lse, 0.7 * (q @ keys[0]), atol=1e-12)
    out0, lse0 = sa.sparse_mla_row(np.zeros((H, D)), keys, 0.7, Dl)
    assert np.allclose(out0, np.broadcast_to(keys[:, :Dl].mean(0), (H, Dl)), atol=1e-15)
    assert np.allclose(lse0, np.log(5.0), atol=1e-15)


def test_mla_lse_and_order_invariance():
    rng = np.random.default_rng(13)
    H, D, Dl = 5, 12, 8
    q = rng.standard_normal((H, D))
    keys = rng.standard_normal((30, D))
    out, lse = sa.sparse_mla_row(q, keys, 1.3, Dl)
    assert np.allclose(lse, scipy.special.logsumexp(1.3 * q @ keys.T, axis=1), atol=1e-12)
    perm = rng.permutation(30)
    out2, lse2 = sa.sparse_mla_row(q, keys[perm], 1.3, Dl)
    assert np.allclose(out, out2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)


def test_pipeline_skips_empty_slots():
    rng = np.random.default_rng(14)
    kv = rng.standard_normal((20, 6)).astype(np.float32)
    q = rng.standard_normal((1, 2, 6)).astype(np.float32)
    a = pl.sparse_mla_rows([0], [np.array([3, 9, -1, -1])], q, "f32", kv, "f32", None, 0.5, 4)
    b = pl.sparse_mla_rows([0], [np.array([9, 3])], q, "f32", kv, "f32", None, 0.5, 4)
    assert np.allclose(a[0], b[0], atol=1e-15) and np.allclose(a[1], b[1], atol=1e-15)


# ------------------------------------------- end to end: context parallelism

def _run_rank(cu, cp, r, qs_all, qi_all, w_all, kv, ki, topk, scale, Dl):
    """One rank: metadata, all-gather stand-in + rerange, then its queries."""
    T = int(cu[-1])
    m = rr.split_metadata(cu, cp, r)
    slot = max(rr.local_count(T, cp, x) for x in range(cp))
    kv_full = rr.rerange(rr.rank_concat(kv, cp, slot), T, cp, slot)
    ki_full = rr.rerange(rr.rank_concat(ki, cp, slot), T, cp, slot)
    g = m["global_idx"]
    rows = range(g.size)
    sel = pl.indexer_topk_rows(rows, m, rr.split_rows(qi_all, cp, r), "f32",
                               rr.split_rows(w_all, cp, r), ki_full, "f32", None, topk)
    idx = [s["topk_idx"] for s in sel]
    out, lse = pl.sparse_mla_rows(rows, idx, rr.split_rows(qs_all, cp, r), "f32",
                                  kv_full, "f32", None, scale, Dl)
    return g, idx, out, lse


def test_context_parallel_invariance_and_page_example():
    # Local queries against the complete KV give the same outputs as running
    # without context parallelism (section 4 part 3, step C); checked on the
    # page's 8-token / 4-rank layout and on a ragged multi-request batch.
    rng = np.random.default_rng(21)
    H, Dl, Dr, Hi, Di = 4, 16, 8, 2, 8
    for cu in ([0, 8], [0, 13, 14, 40]):
        T = cu[-1]
        qs = rng.standard_normal((T, H, Dl + Dr)).astype(np.float32)
        qi = rng.standard_normal((T, Hi, Di)).astype(np.float32)
        w = rng.standard_normal((T, Hi)).astype(np.float32)
        kv = rng.standard_normal((T, Dl + Dr)).astype(np.float32)
        ki = rng.standard_normal((T, Di)).astype(np.float32)
        topk = 5
        g1, idx1, out1, lse1 = _run_rank(cu, 1, 0, qs, qi, w, kv, ki, topk, 0.3, Dl)
        assert g1.tolist() == list(range(T))
        for cp in (2, 4):
            for r in range(cp):
                g, idx, out, lse = _run_rank(cu, cp, r, qs, qi, w, kv, ki, topk, 0.3, Dl)
                for i, gg in enumerate(g.tolist()):
                    assert np.array_equal(idx[i], idx1[gg])
                    assert np.array_equal(out[i], out1[gg])
                    assert np.array_equal(lse[i], lse1[gg])


def test_future_keys_do_not_matter():
    rng = np.random.default_rng(22)
    T, H, D, Hi, Di = 30, 3, 12, 2, 4
    qs = rng.standard_normal((T, H, D)).astype(np.float32)
    qi = rng.standard_normal((T, Hi, Di)).astype(np.float32)
    w = rng.standard_normal((T, Hi)).astype(np.float32)
    kv = rng.standard_normal((T, D)).astype(np.float32)
    ki = rng.standard_normal((T, Di)).astype(np.float32)
    base = _run_rank([0, T], 1, 0, qs, qi, w, kv, ki, 6, 0.5, 8)
    kv2, ki2 = kv.copy(), ki.copy()
    kv2[20:] = 100.0
    ki2[20:] = -7.0
    pert = _run_rank([0, T], 1, 0, qs, qi, w, kv2, ki2, 6, 0.5, 8)
    assert np.array_equal(base[2][:20], pert[2][:20])
    assert not np.array_equal(base[2][20:], pert[2][20:])


def test_decode_metadata_reading():
    m = pl.decode_metadata([5, 1, 64])
    assert m["q_req"].tolist() == [0, 1, 2]
    assert m["kv_start"].tolist() == [0, 0, 0] and m["kv_len"].tolist() == [5, 1, 64]
