"""Runs one rank's hot path on the GPU through the C ABI (test helper).

Inputs come from ``synth``; every step runs in libds32cp.so.  The
all-gather is stood in for by the split kernel itself: each rank's own
rows are gathered into its slot of a rank-concatenated buffer whose padding
is filled with all-ones bytes (NaN for bf16/fp32/e4m3fn), so a kernel that
read padding would be caught.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import deepseek_v3_context_amd as ds

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, fmt: str) -> torch.Tensor:
    if fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.bfloat16)
    if fmt == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV).view(torch.float8_e4m3fn)
    raise ValueError(fmt)


def raw_bytes(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def rank_concat_on_gpu(logical: torch.Tensor, cu: torch.Tensor, T: int, cp: int):
    """All-gather stand-in: slot r holds rank r's own rows (split kernel)."""
    slot = ds.cp_local_count(T, cp, 0)
    cat = torch.empty((cp * slot,) + tuple(logical.shape[1:]), dtype=logical.dtype, device=DEV)
    cat.view(torch.uint8).fill_(0xFF)
    for r in range(cp):
        n = ds.cp_local_count(T, cp, r)
        if n:
            ds.cp_split_metadata(cu, T, cp, r, rows_src=logical,
                                 out={"rows": cat[r * slot: r * slot + n]})
    return cat, slot


def run_prefill(wl, inp: dict, want_scores: bool = True) -> dict:
    T, cp, r = wl.num_tokens, wl.cp_size, wl.cp_rank
    say(f"[gpu] prefill {wl.name}: T={T} cp={cp} rank={r}")
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    ids = torch.from_numpy(inp["input_ids"]).to(DEV)
    kv_l = to_dev(inp["kv"], wl.kv_fmt)
    ki_l = to_dev(inp["k_idx"], wl.kv_fmt)
    kv_scale = None if inp["kv_scale"] is None else torch.from_numpy(inp["kv_scale"]).to(DEV)
    ki_scale = None if inp["k_idx_scale"] is None else torch.from_numpy(inp["k_idx_scale"]).to(DEV)
    kv_cat, slot = rank_concat_on_gpu(kv_l, cu, T, cp)
    ki_cat, _ = rank_concat_on_gpu(ki_l, cu, T, cp)

    meta = ds.cp_split_metadata(cu, T, cp, r, rows_src=ids)
    kv = ds.kv_rerange(kv_cat, slot, T, cp)
    ki = ds.kv_rerange(ki_cat, slot, T, cp)
    q_idx = to_dev(inp["q_idx"], wl.act_fmt)
    w = torch.from_numpy(inp["w"]).to(DEV)
    q = to_dev(inp["q"], wl.act_fmt)
    idx, score = ds.indexer_topk(q_idx, w, ki, meta["kv_start"], meta["kv_len"], T, wl.topk,
                                 k_scale=ki_scale, want_score=True)
    out, lse = ds.sparse_mla_prefill(q, kv, idx, wl.scale, wl.d_latent, kv_scale=kv_scale)
    res = {}
    if want_scores:
        res["scores"] = ds.indexer_scores(q_idx, w, ki, meta["kv_start"], meta["kv_len"], T,
                                          k_scale=ki_scale)
    torch.cuda.synchronize()
    say(f"[gpu] prefill {wl.name}: done")
    res.update({k: v.cpu().numpy() for k, v in meta.items()})
    res.update({"kv_bytes": raw_bytes(kv), "ki_bytes": raw_bytes(ki),
                "kv_cat_bytes": raw_bytes(kv_cat), "slot": slot,
                "topk_idx": idx.cpu().numpy(), "topk_score": score.cpu().numpy(),
                "out": out.float().cpu().numpy(), "lse": lse.cpu().numpy()})
    if want_scores:
        res["scores"] = res["scores"].cpu().numpy()
    return res


def run_decode(wl, inp: dict, want_scores: bool = True) -> dict:
    say(f"[gpu] decode {wl.name}: {wl.n_req} requests, pool rows {inp['pool_rows']}")
    lengths = torch.from_numpy(inp["lengths"]).to(DEV)
    meta = ds.decode_metadata(lengths)
    table = torch.from_numpy(inp["page_table"]).to(DEV)
    ki = to_dev(inp["k_idx"], wl.kv_fmt)
    kv = to_dev(inp["kv"], wl.kv_fmt)
    q_idx = to_dev(inp["q_idx"], wl.act_fmt)
    w = torch.from_numpy(inp["w"]).to(DEV)
    q = to_dev(inp["q"], wl.act_fmt)
    kv_scale = None if inp["kv_scale"] is None else torch.from_numpy(inp["kv_scale"]).to(DEV)
    ki_scale = None if inp["k_idx_scale"] is None else torch.from_numpy(inp["k_idx_scale"]).to(DEV)
    max_len = int(inp["lengths"].max())
    idx, score = ds.indexer_topk(q_idx, w, ki, meta["kv_start"], meta["kv_len"], max_len,
                                 wl.topk, q_req=meta["q_req"], page_table=table,
                                 page_size=wl.page_size, k_scale=ki_scale, want_score=True)
    out, lse = ds.sparse_mla_decode(q, kv, idx, wl.scale, wl.d_latent, kv_scale=kv_scale)
    res = {}
    if want_scores:
        res["scores"] = ds.indexer_scores(q_idx, w, ki, meta["kv_start"], meta["kv_len"],
                                          max_len, q_req=meta["q_req"], page_table=table,
                                          page_size=wl.page_size, k_scale=ki_scale)
    out_p, lse_p = ds.sparse_mla_prefill(q, kv, idx, wl.scale, wl.d_latent, kv_scale=kv_scale)
    torch.cuda.synchronize()
    say(f"[gpu] decode {wl.name}: done")
    res.update({"topk_idx": idx.cpu().numpy(), "topk_score": score.cpu().numpy(),
                "out": out.float().cpu().numpy(), "lse": lse.cpu().numpy(),
                "out_prefill_kernel": out_p.float().cpu().numpy(),
                "lse_prefill_kernel": lse_p.cpu().numpy()})
    if want_scores:
        res["scores"] = res["scores"].cpu().numpy()
    return res
