#!/usr/bin/env python3
"""Benchmark: one context-parallel rank's sparse-attention step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM:

  prefill: cp_split_metadata (+ row gather of the input token ids),
           kv_rerange of the latent KV and of the indexer keys,
           indexer scores + top-k, sparse MLA (prefill kernel);
  decode:  indexer_topk (scores + top-k in one call) on the paged pool,
           sparse MLA (decode).

After the W warm-up steps, untimed steps keep running for a short settle
time (200 ms by default): a cold MI355X runs the first tens of milliseconds
of work at a visibly lower clock.  A HIP event pair costs a few microseconds
of device time, so events stay out of the calls that are not being
measured: a first pass of K steps brackets every call with events (the
per-kernel table, and which kernel dominates); the timed region then runs
K steps with events around the dominant call only, and its wall clock
between two device synchronisations gives the step time.  The printed JSON carries the roofline of the dominant
kernel, taken from the timed region, and the CPU oracle's rate on a bounded
sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--settle-ms MS]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/s per GPU (indexer+top-k+sparse MLA); % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_t65536_cp8_fp8")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="after the warm-up steps, keep running untimed steps for at least this "
                         "long so that the GPU clocks have ramped (0 = off)")
    ap.add_argument("--all-ranks", action="store_true",
                    help="prefill: after the measurement, also time the step on every rank's "
                         "share under both split modes (round-robin, and the in-sequence split "
                         "it replaces) and report the per-rank spread (rank_balance)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    return ap.parse_args()


class Timed:
    """HIP-event timing of named calls on the current stream (of every call,
    or of the calls named in `only`; the others run unbracketed)."""

    def __init__(self, torch, only=None):
        self.torch = torch
        self.only = only
        self.events = {}

    def run(self, name, fn):
        if self.only is not None and name not in self.only:
            fn()
            return
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.events.setdefault(name, []).append((s, e))

    def avg_ms(self):
        return {k: sum(s.elapsed_time(e) for s, e in v) / len(v) for k, v in self.events.items()}


def rank_max_kv_len(cu_seqlens, cp, r):
    """Longest causal key range of rank r's queries: per request, the
    rank's last token g (g = r mod cp) sees positions cu[b] .. g."""
    best = 0
    cu = [int(x) for x in cu_seqlens]
    for lo, hi in zip(cu[:-1], cu[1:]):
        if hi <= lo:
            continue
        g = hi - 1 - ((hi - 1 - r) % cp)
        if g >= lo:
            best = max(best, g - lo + 1)
    return best


def in_seq_max_kv_len(cu_seqlens, cp, r):
    """Longest causal key range of rank r's queries under the in-sequence
    split: per request of L tokens, its chunk r ends at min(L, (r+1) c),
    c = ceil(L / cp)."""
    best = 0
    cu = [int(x) for x in cu_seqlens]
    for lo, hi in zip(cu[:-1], cu[1:]):
        L = hi - lo
        c = -(-L // cp)
        if L - r * c > 0:
            best = max(best, min(L, (r + 1) * c))
    return best


def setup_prefill(wl, torch, ds, dev, split="round-robin"):
    """Inputs and buffers of one rank's prefill step.  `split` picks the
    rank's queries: round-robin (the method) or in-seq (the contiguous
    split it replaces, for the per-rank balance contrast)."""
    import numpy as np
    from synth import draw_prefill

    T, cp, r = wl.num_tokens, wl.cp_size, wl.cp_rank
    cu_host = wl.cu_seqlens()
    if split == "in-seq":
        n = ds.cp_in_seq_local_count(cu_host, cp, r)
    else:
        n = ds.cp_local_count(T, cp, r)
    inp = draw_prefill(wl, n)

    def up(arr, fmt):
        if fmt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        if fmt == "fp8":
            return torch.from_numpy(arr).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(arr).to(dev)

    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    ids = torch.from_numpy(inp["input_ids"]).to(dev)
    kv_l, ki_l = up(inp["kv"], wl.kv_fmt), up(inp["k_idx"], wl.kv_fmt)
    slot = ds.cp_local_count(T, cp, 0)
    # all-gather stand-in: every rank's own rows, rank after rank (built once
    # by the split kernel, outside the timed region)
    kv_cat = torch.empty((cp * slot, wl.d_qk), dtype=kv_l.dtype, device=dev)
    ki_cat = torch.empty((cp * slot, wl.d_idx), dtype=ki_l.dtype, device=dev)
    kv_cat.view(torch.uint8).fill_(0xFF)
    ki_cat.view(torch.uint8).fill_(0xFF)
    for rk in range(cp):
        m = ds.cp_local_count(T, cp, rk)
        if m:
            ds.cp_split_metadata(cu, T, cp, rk, rows_src=kv_l, out={"rows": kv_cat[rk * slot: rk * slot + m]})
            ds.cp_split_metadata(cu, T, cp, rk, rows_src=ki_l, out={"rows": ki_cat[rk * slot: rk * slot + m]})
    del kv_l, ki_l
    st = {
        "n": n, "inp": inp, "cu": cu, "ids": ids, "kv_cat": kv_cat, "ki_cat": ki_cat,
        "slot": slot, "split": split,
        "q_idx": up(inp["q_idx"], wl.act_fmt), "w": torch.from_numpy(inp["w"]).to(dev),
        "q": up(inp["q"], wl.act_fmt),
        "kv_scale": None if inp["kv_scale"] is None else torch.from_numpy(inp["kv_scale"]).to(dev),
        "ki_scale": None if inp["k_idx_scale"] is None else torch.from_numpy(inp["k_idx_scale"]).to(dev),
    }
    i32 = dict(dtype=torch.int32, device=dev)
    B = cu.numel() - 1
    st["meta"] = {"local_cu": torch.empty(B + 1, **i32), "batch_idx": torch.empty(n, **i32),
                  "global_idx": torch.empty(n, **i32), "kv_start": torch.empty(n, **i32),
                  "kv_len": torch.empty(n, **i32), "rows": torch.empty(n, **i32)}
    st["kv"] = torch.empty((T, wl.d_qk), dtype=kv_cat.dtype, device=dev)
    st["ki"] = torch.empty((T, wl.d_idx), dtype=ki_cat.dtype, device=dev)
    # the longest causal range among the rank's queries (host-known from the
    # request lengths): it sizes the score rows and picks the top-k variant
    st["max_len"] = (in_seq_max_kv_len if split == "in-seq" else rank_max_kv_len)(
        inp["cu_seqlens"], cp, r)
    st["scores"] = torch.empty((n, ((st["max_len"] + 63) // 64) * 64), dtype=torch.float32,
                               device=dev)
    st["topk_idx"] = torch.empty((n, wl.topk), **i32)
    st["out"] = torch.empty((n, wl.n_heads, wl.d_latent), dtype=torch.bfloat16 if wl.act_fmt != "f32" else torch.float32, device=dev)
    st["lse"] = torch.empty((n, wl.n_heads), dtype=torch.float32, device=dev)
    need = ds.sparse_mla_prefill_workspace_size(st["kv"].shape[0], st["kv"].dtype)
    st["mla_ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    return st


def prefill_step(wl, ds, st, tm):
    T, cp, r = wl.num_tokens, wl.cp_size, wl.cp_rank
    m = st["meta"]
    if st.get("split") == "in-seq":
        tm.run("cp_split_metadata", lambda: ds.cp_split_metadata_in_seq(st["cu"], T, cp, r, n_local=st["n"], rows_src=st["ids"], out=m))
    else:
        tm.run("cp_split_metadata", lambda: ds.cp_split_metadata(st["cu"], T, cp, r, rows_src=st["ids"], out=m))
    tm.run("kv_rerange(latent)", lambda: ds.kv_rerange(st["kv_cat"], st["slot"], T, cp, out=st["kv"]))
    tm.run("kv_rerange(indexer_k)", lambda: ds.kv_rerange(st["ki_cat"], st["slot"], T, cp, out=st["ki"]))
    tm.run("indexer_scores", lambda: ds.indexer_scores(st["q_idx"], st["w"], st["ki"], m["kv_start"], m["kv_len"], st["max_len"], k_scale=st["ki_scale"], scores=st["scores"]))
    tm.run("topk_select", lambda: ds.topk_select(st["scores"], m["kv_start"], m["kv_len"], st["max_len"], wl.topk, T, topk_idx=st["topk_idx"]))
    tm.run("sparse_mla", lambda: ds.sparse_mla_prefill(st["q"], st["kv"], st["topk_idx"], wl.scale, wl.d_latent, kv_scale=st["kv_scale"], out=st["out"], lse=st["lse"], workspace=st["mla_ws"]))


def setup_decode(wl, torch, ds, dev):
    import numpy as np
    from synth import draw_decode

    inp = draw_decode(wl)

    def up(arr, fmt):
        if fmt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        if fmt == "fp8":
            return torch.from_numpy(arr).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(arr).to(dev)

    n = wl.n_req
    lengths = torch.from_numpy(inp["lengths"]).to(dev)
    max_len = int(inp["lengths"].max())
    st = {"n": n, "inp": inp, "meta": ds.decode_metadata(lengths),
          "table": torch.from_numpy(inp["page_table"]).to(dev),
          "ki": up(inp["k_idx"], wl.kv_fmt), "kv": up(inp["kv"], wl.kv_fmt),
          "q_idx": up(inp["q_idx"], wl.act_fmt), "w": torch.from_numpy(inp["w"]).to(dev),
          "q": up(inp["q"], wl.act_fmt), "max_len": max_len,
          "kv_scale": None if inp["kv_scale"] is None else torch.from_numpy(inp["kv_scale"]).to(dev),
          "ki_scale": None if inp["k_idx_scale"] is None else torch.from_numpy(inp["k_idx_scale"]).to(dev)}
    st["ix_ws"] = torch.empty(ds.indexer_topk_workspace_size(n, max_len), dtype=torch.uint8, device=dev)
    st["topk_idx"] = torch.empty((n, wl.topk), dtype=torch.int32, device=dev)
    st["out"] = torch.empty((n, wl.n_heads, wl.d_latent), dtype=torch.bfloat16, device=dev)
    st["lse"] = torch.empty((n, wl.n_heads), dtype=torch.float32, device=dev)
    st["ws"] = torch.empty(ds.sparse_mla_workspace_size(n, wl.n_heads, wl.d_latent, wl.topk),
                           dtype=torch.uint8, device=dev)
    return st


def decode_step(wl, ds, st, tm):
    m = st["meta"]
    paging = dict(q_req=m["q_req"], page_table=st["table"], page_size=wl.page_size)
    tm.run("indexer_topk", lambda: ds.indexer_topk(st["q_idx"], st["w"], st["ki"], m["kv_start"], m["kv_len"], st["max_len"], wl.topk, k_scale=st["ki_scale"], topk_idx=st["topk_idx"], workspace=st["ix_ws"], **paging))
    tm.run("sparse_mla", lambda: ds.sparse_mla_decode(st["q"], st["kv"], st["topk_idx"], wl.scale, wl.d_latent, kv_scale=st["kv_scale"], out=st["out"], lse=st["lse"], workspace=st["ws"]))


# source files whose kernels each call launches (a counter record is used only
# while these files are unchanged since the counters were taken)
CALL_SOURCES = {"sparse_mla": ("sparse_mla.hip", "common.h"),
                "indexer_scores": ("indexer.hip", "common.h"),
                "topk_select": ("topk.hip", "common.h"),
                "indexer_topk": ("indexer.hip", "topk.hip", "common.h")}


def counted_traffic(call, workload):
    """HBM bytes per launch of `call` from the committed rocprofv3 counter
    record of this workload (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for the latent-KV rerange, a copy of known size).
    None when there is no record or the kernel sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{workload}.txt")
    if call not in CALL_SOURCES or not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in CALL_SOURCES[call]:
        with open(os.path.join(ROOT, "deepseek_v3_context_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()[:16]
    scale, rec = None, None
    with open(path) as fh:
        for line in fh:
            tok = line.split()
            if not tok or tok[0].startswith("#"):
                continue
            if tok[0] == "scale":
                scale = (float(tok[1]), float(tok[2]))
            elif tok[0] == call:
                rec = tok
    if scale is None or rec is None or rec[1] != sha:
        return None
    return int(round((float(rec[2]) * scale[0] + float(rec[3]) * scale[1]) * 1024))


def work_model(wl, kv_len):
    """Algorithmic work per call: causal pairs for the indexer, valid top-k
    pairs for MLA; bytes are the unavoidable HBM traffic of each call."""
    import numpy as np
    kv_len = np.asarray(kv_len, dtype=np.int64)
    n = kv_len.size
    idx_pairs = int(kv_len.sum())
    mla_pairs = int(np.minimum(kv_len, wl.topk).sum())
    act = 4 if wl.act_fmt == "f32" else 2
    kvb = {"f32": 4, "bf16": 2, "fp8": 1}[wl.kv_fmt]
    T = wl.num_tokens if wl.kind == "prefill" else 0
    mla_flops = mla_pairs * 2 * wl.n_heads * (2 * wl.d_latent + wl.d_rope)
    idx_flops = idx_pairs * (2 * wl.h_idx * wl.d_idx + wl.h_idx)
    out = {
        "indexer_scores": {"flops": idx_flops,
                           "bytes": n * wl.h_idx * (wl.d_idx * act + 4)
                           + (T if T else idx_pairs) * wl.d_idx * kvb + idx_pairs * 4},
        "topk_select": {"flops": 0, "bytes": idx_pairs * 4 + n * wl.topk * 4},
        # indexer + top-k in one call (decode): keys and queries read once, the
        # scores written and read back once, the selection written
        "indexer_topk": {"flops": idx_flops,
                         "bytes": n * wl.h_idx * (wl.d_idx * act + 4) + idx_pairs * wl.d_idx * kvb
                         + 2 * idx_pairs * 4 + n * wl.topk * 4},
        "sparse_mla": {"flops": mla_flops,
                       "bytes": n * wl.n_heads * (wl.d_qk * act + wl.d_latent * 2 + 4)
                       + mla_pairs * wl.d_qk * kvb + n * wl.topk * 4},
    }
    if wl.kind == "prefill":
        row = lambda d: d * kvb  # noqa: E731
        out["kv_rerange(latent)"] = {"flops": 0, "bytes": 2 * T * row(wl.d_qk)}
        out["kv_rerange(indexer_k)"] = {"flops": 0, "bytes": 2 * T * row(wl.d_idx)}
        out["cp_split_metadata"] = {"flops": 0, "bytes": n * 4 * 6}
    return out, idx_pairs, mla_pairs


def cpu_baseline(wl, st, kv_len_host, seconds):
    """The CPU oracle, as it stands, on a bounded sample of query rows."""
    import numpy as np
    from oracle import pipeline as opl
    from oracle import round_robin_cp as orr

    # multithreaded BLAS with the thread count it is configured for: the
    # affinity mask can list every CPU of the host while the process's CPU
    # share is smaller (OMP_NUM_THREADS and the like name that share), and
    # raising the BLAS to the mask's size oversubscribes the share
    visible = len(os.sched_getaffinity(0))
    cores, blas = visible, "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
            cores = min(visible, int(info[0].get("num_threads", visible)))
    except Exception:  # pragma: no cover
        pass
    inp = st["inp"]
    n = st["n"]
    if wl.kind == "prefill":
        meta = orr.split_metadata(inp["cu_seqlens"], wl.cp_size, wl.cp_rank)
        paging = {}
    else:
        meta = opl.decode_metadata(inp["lengths"])
        paging = {"page_table": inp["page_table"], "page_size": wl.page_size}
    order = np.random.default_rng(0).permutation(n)
    done, t0 = 0, time.perf_counter()
    for j in order:
        sel = opl.indexer_topk_rows([j], meta, inp["q_idx"], wl.act_fmt, inp["w"], inp["k_idx"],
                                    wl.kv_fmt, inp["k_idx_scale"], wl.topk, **paging)
        opl.sparse_mla_rows([j], [sel[0]["topk_idx"]], inp["q"], wl.act_fmt, inp["kv"],
                            wl.kv_fmt, inp["kv_scale"], wl.scale, wl.d_latent)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query tokens/s", "cores": int(cores),
            "cpus_visible": visible, "kind": "oracle", "blas": blas,
            "label": "plain NumPy oracle, not an optimized CPU baseline",
            "sample": f"{done} of {n} query rows (seeded random order over the rank's "
                      f"queries), indexer + top-k + sparse MLA in float64 NumPy, {dt:.1f} s"}


def own_kv_cache_write(wl, torch, ds, st, dev, steps):
    """The rank keeping its own tokens' latent KV and indexer keys in a paged
    pool (64-row pages, the decode pool's), after the timed region and
    outside the step.  `steps` back-to-back calls of each sit between one
    HIP event pair (a pair per call would mostly time the events, the call
    being a few microseconds).  The host takes longer to issue a call than
    the device to run it, so a bounded spin kernel holds the stream until
    every call is queued: the pair then times the device running them back
    to back.  Bytes per call: each own row read once and written once (the
    fp8 write: bf16 rows read, e4m3fn codes and a scale per row written)."""
    from synth import draw_page_table

    print("[bench] own-KV cache write", file=sys.stderr, flush=True)
    m = st["meta"]
    lcu = m["local_cu"].cpu().numpy()
    n = int(lcu[-1])
    table, pool_rows = draw_page_table(lcu[1:] - lcu[:-1], 64, seed=wl.seed)
    table_d = torch.from_numpy(table).to(dev)
    r, slot = wl.cp_rank, st["slot"]
    srcs = {"kv_cache_write(latent)": st["kv_cat"][r * slot: r * slot + n],
            "kv_cache_write(indexer_k)": st["ki_cat"][r * slot: r * slot + n]}
    pools = {k: torch.empty((pool_rows,) + tuple(v.shape[1:]), dtype=v.dtype, device=dev)
             for k, v in srcs.items()}
    # fp8 on write: the rank's own rows in bf16 (as its projections produce
    # them; seeded N(0,1)/sqrt(D) values of the rows' shape) encoded into
    # pools with a scale per row
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    fp8_srcs = {"kv_cache_write_fp8(latent)": wl.d_qk, "kv_cache_write_fp8(indexer_k)": wl.d_idx}
    fp8_rows = {k: (torch.randn((n, d), generator=g, device=dev) * d ** -0.5).bfloat16()
                for k, d in fp8_srcs.items()}
    fp8_pools = {k: (torch.empty((pool_rows, d), dtype=torch.uint8, device=dev),
                     torch.empty(pool_rows, dtype=torch.float32, device=dev))
                 for k, d in fp8_srcs.items()}

    def timed(call):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(60000 * steps)   # ~25 us of device time per queued call
        ev0.record()
        for _ in range(steps):
            call()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    per_call, nbytes = {}, {}
    for k, v in srcs.items():
        per_call[k] = timed(lambda: ds.kv_cache_write(v, m["batch_idx"], m["local_cu"], table_d,
                                                      64, pools[k]))
        nbytes[k] = 2 * n * v.element_size() * v[0].numel() if n else 0
    for k, d in fp8_srcs.items():
        codes, scales = fp8_pools[k]
        per_call[k] = timed(lambda: ds.kv_cache_write_fp8(fp8_rows[k], m["batch_idx"], m["local_cu"],
                                                          table_d, 64, codes, scales))
        nbytes[k] = n * (2 * d + d + 4)       # bf16 rows read, codes and scales written
    out = {}
    for k, ms in per_call.items():
        gbs = nbytes[k] / (ms * 1e-3) / 1e9
        out[k] = {"avg_us": round(ms * 1e3, 2), "bytes": nbytes[k], "gbs": round(gbs, 1),
                  "bound": "hbm", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


# The dense projections around the path at DeepSeek-V3.2's dimensions
# (hidden 7168, q compression 1536, 128 heads x (128 nope + 64 rope), latent
# 512, value head 128; indexer 64 x 128): name -> (N, K, batch); M is the
# rank's token count.
PROJECTIONS = {
    "mla_q_down": (1536, 7168, 1),
    "mla_q_up": (128 * 192, 1536, 1),
    "mla_q_absorb": (512, 128, 128),        # per head, into the latent part of q
    "indexer_wq_b": (64 * 128, 1536, 1),
    "indexer_w_k": (128, 7168, 1),
    "mla_value_up": (128, 512, 128),        # per head, O_latent . W_UV
    "o_proj": (7168, 128 * 128, 1),
}


def projections(wl, torch, ds, n, steps):
    """Each projection GEMM on the rank's n tokens with seeded synthetic
    weights (no trained weights), outside the step: `steps` back-to-back
    calls between one event pair, the stream held by a spin kernel until
    all are queued.  The per-head products run on the strided in-place views
    the path uses (q_up's nope part -> the latent part of the 576-wide MLA
    query; O_latent -> the value rows)."""
    print("[bench] projections", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(wl.seed)

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, generator=g, device=dev) * scale).bfloat16()

    out = {}
    for name, (N, K, batch) in PROJECTIONS.items():
        if name == "mla_q_absorb":
            q_up = rnd(n, 128, 192)
            a, w = q_up[:, :, :128].transpose(0, 1), rnd(128, 512, 128, scale=128 ** -0.5)
            q_mla = torch.empty((n, 128, 576), dtype=torch.bfloat16, device=dev)
            c = q_mla[:, :, :512].transpose(0, 1)
        elif name == "mla_value_up":
            a, w = rnd(n, 128, 512).transpose(0, 1), rnd(128, 128, 512, scale=512 ** -0.5)
            c = torch.empty((n, 128 * 128), dtype=torch.bfloat16, device=dev).view(n, 128, 128).transpose(0, 1)
        else:
            a, w = rnd(n, K), rnd(N, K, scale=K ** -0.5)
            c = torch.empty((n, N), dtype=torch.bfloat16, device=dev)
        need = ds.gemm_bf16_nt_workspace_size(n, N, K, batch)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ds.gemm_bf16_nt(a, w, out=c, workspace=ws)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(60000 * steps)
        ev0.record()
        for _ in range(steps):
            ds.gemm_bf16_nt(a, w, out=c, workspace=ws)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        flops = 2.0 * n * N * K * batch
        tf = flops / (ms * 1e-3) / 1e12
        # algorithmic HBM bytes: A, B and C once each (bf16); below the
        # ridge (peak FLOP/s over peak bytes/s) the product is HBM-bound
        nbytes = 2.0 * (n * K + N * K + n * N) * batch
        gbs = nbytes / (ms * 1e-3) / 1e9
        hbm = flops / nbytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        out[name] = {"M": n, "N": N, "K": K, "batch": batch, "avg_us": round(ms * 1e3, 2),
                     "tflops": round(tf, 1), "gbs": round(gbs, 1), "bytes": int(nbytes),
                     "bound": "hbm" if hbm else "mfma",
                     "frac": round(gbs / PEAK_HBM_GBS if hbm else tf / PEAK_BF16_TFLOPS, 4),
                     "splits": 1 if need == 0 else need // (4 * n * N * batch)}
        del a, w, c, ws
    torch.cuda.empty_cache()
    return out


def cold_steps(wl, torch, ds, st, step, steps):
    """The step with the Infinity Cache (MALL) flushed before each one: a
    512 MB scratch write between steps, outside the events; one event pair
    around every step."""
    print("[bench] cold-cache steps", file=sys.stderr, flush=True)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    none = Timed(torch, only=())
    ms = []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        step(wl, ds, st, none)
        ev1.record()
        torch.cuda.synchronize()
        ms.append(ev0.elapsed_time(ev1))
    del flush
    ms.sort()
    return {"ms_per_step_median": round(ms[len(ms) // 2], 4), "ms_per_step_mean": round(sum(ms) / len(ms), 4),
            "steps": steps, "flush": "512 MB device write before every step, outside the events"}


def rank_balance(wl, torch, ds, dev, args, split):
    """The step on every rank's share of the same prefill under one split
    mode, each rank set up on its own, warmed up and timed like the main
    measurement (K steps between two device synchronisations, no events).
    spread = (max - min) / mean of the per-rank step times.  The in-seq
    step runs the same calls as the round-robin one (its rerange call
    moves the same bytes as the in-seq mode's own would); only the split,
    and so each rank's queries and causal ranges, differ."""
    import dataclasses

    ms, nq, ipairs, mpairs = [], [], [], []
    for r in range(wl.cp_size):
        print(f"[bench] rank balance ({split}): rank {r}", file=sys.stderr, flush=True)
        wr = dataclasses.replace(wl, cp_rank=r)
        st = setup_prefill(wr, torch, ds, dev, split=split)
        none = Timed(torch, only=())
        t_end = time.perf_counter() + max(args.settle_ms, 0.0) * 1e-3
        for i in range(max(args.warmup, 1)):
            prefill_step(wr, ds, st, none)
        while time.perf_counter() < t_end:
            prefill_step(wr, ds, st, none)
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            prefill_step(wr, ds, st, none)
        torch.cuda.synchronize()
        ms.append(round((time.perf_counter() - t0) / args.steps * 1e3, 4))
        nq.append(st["n"])
        kl = st["meta"]["kv_len"].cpu().long()
        ipairs.append(int(kl.sum()))
        mpairs.append(int(kl.clamp(max=wl.topk).sum()))
        del st
        torch.cuda.empty_cache()
    mean = sum(ms) / len(ms)
    return {"split": split, "ms_per_step": ms, "queries": nq, "indexer_pairs": ipairs,
            "mla_pairs": mpairs, "spread": round((max(ms) - min(ms)) / mean, 4)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one context-parallel rank on one GPU; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported: the library has no "
              f"multi-GPU path, and how the step would shard is described, not implemented.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import deepseek_v3_context_amd as ds
    from synth import get

    wl = get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] setting up {wl.name}", file=sys.stderr, flush=True)
    if wl.kind == "prefill":
        st = setup_prefill(wl, torch, ds, dev)
        step = prefill_step
    else:
        st = setup_decode(wl, torch, ds, dev)
        step = decode_step
    torch.cuda.synchronize()

    warm = Timed(torch, only=())
    for _ in range(args.warmup):
        step(wl, ds, st, warm)
    torch.cuda.synchronize()
    # clock settle: a cold GPU runs the first tens of milliseconds of work
    # well below its steady clock; keep at most 8 steps queued so that the
    # host clock tracks the device's
    settle_steps, t_settle = 0, time.perf_counter()
    while args.settle_ms > 0 and time.perf_counter() - t_settle < args.settle_ms * 1e-3:
        step(wl, ds, st, warm)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    if wl.kind == "prefill":
        kv_len_host = st["meta"]["kv_len"].cpu().numpy()
    else:
        kv_len_host = st["inp"]["lengths"]
    print(f"[bench] per-call pass, {args.steps} steps", file=sys.stderr, flush=True)
    calls = Timed(torch)
    for _ in range(args.steps):
        step(wl, ds, st, calls)
    torch.cuda.synchronize()
    per_call = calls.avg_ms()
    dom = max(per_call, key=per_call.get)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    tm = Timed(torch, only=(dom,))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(wl, ds, st, tm)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    model, idx_pairs, mla_pairs = work_model(wl, kv_len_host)
    kernels = {}
    for name, ms in per_call.items():
        w = model.get(name, {"flops": 0, "bytes": 0})
        kernels[name] = {"avg_us": round(ms * 1e3, 2),
                         "tflops": round(w["flops"] / (ms * 1e-3) / 1e12, 2),
                         "gbs": round(w["bytes"] / (ms * 1e-3) / 1e9, 1)}
    dw = model[dom]
    d_ms = tm.avg_ms()[dom]
    # prefill indexer and MLA are dense contractions over tiles (MFMA-bound);
    # decode and the permutations stream HBM
    if wl.kind == "prefill" and dom in ("sparse_mla", "indexer_scores"):
        ach = dw["flops"] / (d_ms * 1e-3) / 1e12
        roof = {"kernel": dom, "avg_us": round(d_ms * 1e3, 2), "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": counted_traffic(dom, wl.name)}
    else:
        ach = dw["bytes"] / (d_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "avg_us": round(d_ms * 1e3, 2), "bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": counted_traffic(dom, wl.name)}
    n = st["n"]
    ms_step = elapsed / args.steps * 1e3
    line = {
        "metric": METRIC, "value": round(n * args.steps / elapsed, 1),
        "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.act_fmt == "bf16" else wl.act_fmt,
        "data": "synthetic (seeded N(0,1)/sqrt(dim) activations; no trained weights)",
        "config": {"workload": wl.name, "kind": wl.kind, "queries": n,
                   "num_tokens": wl.num_tokens if wl.kind == "prefill" else int(np.sum(kv_len_host)),
                   "cp_size": wl.cp_size, "cp_rank": wl.cp_rank, "topk": wl.topk,
                   "heads": wl.n_heads, "d_latent": wl.d_latent, "d_rope": wl.d_rope,
                   "indexer": f"{wl.h_idx}x{wl.d_idx}", "kv_format": wl.kv_fmt,
                   "indexer_pairs": idx_pairs, "mla_pairs": mla_pairs},
        "roofline": roof,
        "kernels": kernels,
        "untimed": {"warmup_steps": args.warmup, "settle_steps": settle_steps,
                    "settle_ms": round(settle_ms, 1), "per_call_pass_steps": args.steps},
        "kernel_timing": "kernels: separate pass, HIP events around every call; "
                         "roofline: timed region, events around the dominant call only",
        "kernel_gbs": "algorithmic bytes per call / time; sparse_mla counts every selected "
                      "row once per query that selects it (gathered bytes, not HBM traffic)",
    }
    if wl.kind == "decode":
        line["cold_cache"] = cold_steps(wl, torch, ds, st, step, args.steps)
    if wl.kind == "prefill":
        line["outside_step"] = own_kv_cache_write(wl, torch, ds, st, dev, args.steps)
        line["projections"] = projections(wl, torch, ds, st["n"], args.steps)
        if args.all_ranks:
            line["rank_balance"] = {mode: rank_balance(wl, torch, ds, dev, args, mode)
                                    for mode in ("round-robin", "in-seq")}
    if args.cpu_seconds > 0:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, st, kv_len_host, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
