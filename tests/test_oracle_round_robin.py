"""Pins of the round-robin split / metadata / rerange oracle.

Each test ties the oracle to something other than itself: the worked
examples the blog post prints ("[DeepSeek v3.2] 上下文并行详解", section 4
parts 1 and 3; fixtures under tests/golden/), closed forms derived by hand,
numpy's searchsorted, and round-trip / partition invariants.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import round_robin_cp as rr
from synth import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def test_page_example_8_tokens_on_4_ranks():
    g = _golden("cp4_8tokens.json")
    T, cp = g["num_tokens"], g["cp_size"]
    for r, owned in g["ownership"].items():
        assert rr.rank_global_ids(T, cp, int(r)).tolist() == owned
        assert rr.split_metadata([0, T], cp, int(r))["global_idx"].tolist() == owned
    tokens = np.arange(T, dtype=np.int64)
    concat = rr.rank_concat(tokens, cp)
    assert concat.tolist() == g["rank_concatenated_order"]
    assert rr.rerange(concat, T, cp, slot_rows=2).tolist() == g["logical_order"]
    assert rr.rank_global_ids(T, cp, 1).tolist() == g["rank1_queries"]


def test_page_causal_example():
    # T5 attends to T0..T4; the reading adopted is inclusive of itself.
    g = _golden("cp4_8tokens.json")
    q = g["causal_example"]["query"]
    meta = rr.split_metadata([0, g["num_tokens"]], g["cp_size"], q % g["cp_size"])
    j = meta["global_idx"].tolist().index(q)
    keys = set(range(meta["kv_start"][j], meta["kv_start"][j] + meta["kv_len"][j]))
    assert set(g["causal_example"]["attends_to_earlier"]) <= keys
    assert keys == set(g["causal_example"]["attends_to_earlier"]) | {q}


def test_page_example_8000_tokens_on_8_ranks():
    g = _golden("cp8_8000tokens.json")
    T, cp = g["num_tokens"], g["cp_size"]
    for r in range(cp):
        assert rr.local_count(T, cp, r) == g["tokens_per_rank"]
    ranges = rr.in_seq_split_ranges(T, cp)
    for r, (lo, hi) in g["in_seq_split_printed_ranges"].items():
        assert ranges[int(r)] == (lo, hi)
    ex = g["two_request_example"]
    got = [rr.in_seq_split_ranges(L, cp)[0] for L in ex["lengths"]]
    assert [list(x) for x in got] == ex["rank0_ranges"]


@pytest.mark.parametrize("T", [0, 1, 2, 3, 7, 8, 9, 63, 64, 65, 1000, 8001])
@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_count_balance_and_closed_form(T, cp):
    counts = [rr.local_count(T, cp, r) for r in range(cp)]
    assert sum(counts) == T
    assert max(counts) - min(counts) <= 1          # balance claim, section 4 part 3
    for r in range(cp):
        assert counts[r] == max(0, math.ceil((T - r) / cp))


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.kind == "prefill"])
def test_count_balance_on_workloads(name):
    w = WORKLOADS[name]
    counts = [rr.local_count(w.num_tokens, w.cp_size, r) for r in range(w.cp_size)]
    assert max(counts) - min(counts) <= 1
    assert sum(counts) == w.num_tokens


def test_ranks_partition_the_tokens():
    T, cp = 1237, 8
    seen = np.concatenate([rr.rank_global_ids(T, cp, r) for r in range(cp)])
    assert sorted(seen.tolist()) == list(range(T))


def test_six_request_rank5_metadata_closed_form():
    # Requests {8000, 800, 5, 3000, 1500, 12000}: cu = [0, 8000, 8800, 8805,
    # 11805, 13305, 25305].  Rank 5 of 8 owns g = 5 + 8j, so the number of its
    # tokens below x is ceil((x - 5) / 8) for x > 5:
    #   8000 -> 1000, 8800 -> 1100, 8805 -> 1100 (the 5-token request falls
    #   between two rank-5 tokens), 11805 -> 1475, 13305 -> 1663,
    #   25305 -> 3163.
    cu = [0, 8000, 8800, 8805, 11805, 13305, 25305]
    meta = rr.split_metadata(cu, 8, 5)
    assert meta["local_cu"].tolist() == [0, 1000, 1100, 1100, 1475, 1663, 3163]
    assert np.bincount(meta["batch_idx"], minlength=6).tolist() == \
        [1000, 100, 0, 375, 188, 1500]


def _random_cu(rng, n_req, max_len, allow_empty=True):
    lens = rng.integers(0 if allow_empty else 1, max_len + 1, size=n_req)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("seed", range(6))
def test_metadata_properties(seed):
    rng = np.random.default_rng(seed)
    cu = _random_cu(rng, int(rng.integers(1, 7)), 60)
    T = int(cu[-1])
    for cp in (1, 2, 3, 8):
        for r in range(cp):
            m = rr.split_metadata(cu, cp, r)
            g = m["global_idx"].astype(np.int64)
            assert (g % cp == r).all()
            assert np.array_equal(g, np.arange(r, T, cp))
            # request of each token: library routine on the offsets
            assert np.array_equal(m["batch_idx"],
                                  np.searchsorted(cu, g, side="right") - 1)
            assert np.array_equal(m["kv_start"], cu[m["batch_idx"]])
            # causal range ends at the query itself (inclusive reading)
            assert np.array_equal(m["kv_start"] + m["kv_len"] - 1, g)
            assert (m["kv_len"] >= 1).all()
            # recomputed offsets: per-request counts of the rank's tokens
            per_req = np.diff(m["local_cu"])
            assert np.array_equal(per_req, np.bincount(m["batch_idx"],
                                                       minlength=len(cu) - 1))
            assert m["local_cu"][0] == 0 and m["local_cu"][-1] == g.size


def test_rejects_bad_offsets():
    with pytest.raises(ValueError):
        rr.split_metadata([1, 5], 2, 0)
    with pytest.raises(ValueError):
        rr.split_metadata([0, 5, 3], 2, 0)
    with pytest.raises(ValueError):
        rr.rank_global_ids(5, 2, 2)


@pytest.mark.parametrize("T,cp,extra", [(8, 4, 0), (13, 4, 0), (13, 4, 3),
                                        (1, 8, 0), (0, 3, 0), (1000, 8, 1)])
def test_rerange_round_trip_and_padding_never_read(T, cp, extra):
    rng = np.random.default_rng(T * 31 + cp)
    x = rng.standard_normal((T, 5)).astype(np.float32)
    slot = (max(rr.local_count(T, cp, r) for r in range(cp)) if T else 0) + extra
    concat = rr.rank_concat(x, cp, slot_rows=slot)     # padding is NaN
    assert concat.shape[0] == cp * slot
    back = rr.rerange(concat, T, cp, slot)
    assert np.array_equal(back, x)                     # bit-exact, no NaN read
    # the split of the reranged buffer is again each rank's slot
    for r in range(cp):
        n = rr.local_count(T, cp, r)
        assert np.array_equal(rr.split_rows(back, cp, r), concat[r * slot: r * slot + n])


def test_rerange_bytes_rows():
    rng = np.random.default_rng(5)
    x = rng.integers(0, 256, size=(77, 576), dtype=np.uint8)
    concat = rr.rank_concat(x, 8)
    assert np.array_equal(rr.rerange(concat, 77, 8, concat.shape[0] // 8), x)


# ------------------------------------------------ in-sequence split (contrast)

def test_in_seq_split_page_example_8000_tokens_on_8_ranks():
    # section 4 part 1: rank r of 8 takes tokens 1000r .. 1000r + 999
    g = _golden("cp8_8000tokens.json")
    T, cp = g["num_tokens"], g["cp_size"]
    for r, (lo, hi) in g["in_seq_split_printed_ranges"].items():
        m = rr.in_seq_split_metadata([0, T], cp, int(r))
        assert m["global_idx"].tolist() == list(range(lo, hi + 1))
        assert m["local_cu"].tolist() == [0, hi - lo + 1]
        assert m["kv_len"].tolist() == list(range(lo + 1, hi + 2))   # causal, inclusive
    for r in range(cp):
        assert rr.in_seq_split_metadata([0, T], cp, r)["global_idx"].size == g["tokens_per_rank"]


def test_in_seq_split_page_two_request_example():
    # same section: requests of 8000 and 800 tokens; rank 0 handles request
    # A's tokens 0..999 and request B's tokens 0..99
    g = _golden("cp8_8000tokens.json")
    ex = g["two_request_example"]
    cu = [0, ex["lengths"][0], ex["lengths"][0] + ex["lengths"][1]]
    m = rr.in_seq_split_metadata(cu, g["cp_size"], 0)
    (a_lo, a_hi), (b_lo, b_hi) = ex["rank0_ranges"]
    want = list(range(a_lo, a_hi + 1)) + [cu[1] + p for p in range(b_lo, b_hi + 1)]
    assert m["global_idx"].tolist() == want
    assert m["batch_idx"].tolist() == [0] * (a_hi - a_lo + 1) + [1] * (b_hi - b_lo + 1)
    assert m["kv_start"].tolist() == [0] * (a_hi - a_lo + 1) + [cu[1]] * (b_hi - b_lo + 1)
    # the single-request ranges of the older helper agree with the metadata
    for L in ex["lengths"]:
        for r in range(g["cp_size"]):
            lo, hi = rr.in_seq_split_ranges(L, g["cp_size"])[r]
            got = rr.in_seq_split_metadata([0, L], g["cp_size"], r)["global_idx"].tolist()
            assert got == list(range(lo, hi + 1))


def test_in_seq_split_three_requests_worked_by_hand():
    # lengths 8000, 800, 5 on 8 ranks (the page's imbalance example): chunks
    # of 1000, 100 and 1 tokens; ranks 0..4 get one token of the 5-token
    # request each, ranks 5..7 none; rank 6's tokens are A 6000..6999 and
    # B 600..699.
    cu = [0, 8000, 8800, 8805]
    counts = [rr.in_seq_split_metadata(cu, 8, r)["global_idx"].size for r in range(8)]
    assert counts == [1101] * 5 + [1100] * 3
    m6 = rr.in_seq_split_metadata(cu, 8, 6)
    assert m6["local_cu"].tolist() == [0, 1000, 1100, 1100]
    assert m6["global_idx"].tolist() == list(range(6000, 7000)) + list(range(8600, 8700))
    m4 = rr.in_seq_split_metadata(cu, 8, 4)
    assert m4["global_idx"][-1] == 8804 and m4["kv_len"][-1] == 5


def test_in_seq_split_causal_work_is_unbalanced():
    # one 8000-token request on 8 ranks: rank r's causal pairs are
    # sum_{p = 1000r}^{1000r + 999} (p + 1), from 500 500 (rank 0) to
    # 7 500 500 (rank 7); round-robin gives every rank 3 996 000 - 4 004 000
    for r in range(8):
        m = rr.in_seq_split_metadata([0, 8000], 8, r)
        lo, hi = 1000 * r, 1000 * r + 999
        assert int(m["kv_len"].astype(np.int64).sum()) == (hi + 1) * (hi + 2) // 2 - lo * (lo + 1) // 2
        rrm = rr.split_metadata([0, 8000], 8, r)
        assert 3_996_000 <= int(rrm["kv_len"].astype(np.int64).sum()) <= 4_004_000


@pytest.mark.parametrize("seed", range(6))
def test_in_seq_split_partition_and_contiguity(seed):
    rng = np.random.default_rng(100 + seed)
    cu = _random_cu(rng, int(rng.integers(1, 7)), 60)
    T = int(cu[-1])
    for cp in (1, 2, 3, 8):
        metas = [rr.in_seq_split_metadata(cu, cp, r) for r in range(cp)]
        seen = np.concatenate([m["global_idx"] for m in metas]).astype(np.int64)
        assert sorted(seen.tolist()) == list(range(T))          # each token exactly once
        owner = np.empty(T, dtype=np.int64)
        for r, m in enumerate(metas):
            g = m["global_idx"].astype(np.int64)
            owner[g] = r
            assert np.array_equal(m["batch_idx"], np.searchsorted(cu, g, side="right") - 1)
            assert np.array_equal(m["kv_start"], cu[m["batch_idx"]])
            assert np.array_equal(m["kv_start"] + m["kv_len"] - 1, g)
            per_req = np.diff(m["local_cu"])
            assert np.array_equal(per_req, np.bincount(m["batch_idx"], minlength=len(cu) - 1))
        # along each request the owning rank never decreases, and a rank's
        # tokens of a request are consecutive (one chunk)
        for b in range(len(cu) - 1):
            o = owner[cu[b]: cu[b + 1]]
            assert (np.diff(o) >= 0).all()
