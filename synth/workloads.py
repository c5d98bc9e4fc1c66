"""Named workloads: shapes, formats and seeds.

Shapes follow the pages' own scenarios: an 8000-token prompt on 8 ranks and
requests of 8000 / 800 / 5 tokens ("[DeepSeek v3.2] 上下文并行详解",
section 4 part 1), up to 32 running requests (same page, section 3), the
64K+ sequence band where context parallelism is added ("Model Parallel
Strategy Analysis", step 2 layer 3), 128 MLA heads in total (16 per rank
under 8-way attention TP, "[RFC]: Parallel strategy for Deepseek v3.2 like
models", old implementation).  Latent width 512 + rope 64 and the 64x128
indexer are DeepSeek-V3.2's published dimensions.

``act_fmt`` is the storage of the queries (``q``, ``q_idx``); ``kv_fmt`` the
storage of the latent KV rows and indexer keys: ``"f32"``, ``"bf16"`` or
``"fp8"`` (e4m3fn codes + one fp32 scale per 128 rows).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                       # "prefill" or "decode"
    seed: int
    n_heads: int = 128
    d_latent: int = 512
    d_rope: int = 64
    h_idx: int = 64
    d_idx: int = 128
    topk: int = 2048
    act_fmt: str = "bf16"
    kv_fmt: str = "bf16"
    sm_scale: float | None = None   # default 1/sqrt(d_latent + d_rope)
    # prefill
    seqlens: tuple = ()
    cp_size: int = 1
    cp_rank: int = 0
    # decode
    n_req: int = 0
    len_lo: int = 0
    len_hi: int = 0
    page_size: int = 64
    description: str = field(default="", compare=False)

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def scale(self) -> float:
        if self.sm_scale is not None:
            return float(self.sm_scale)
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def num_tokens(self) -> int:
        return int(sum(self.seqlens))

    def cu_seqlens(self) -> list[int]:
        out = [0]
        for s in self.seqlens:
            out.append(out[-1] + int(s))
        return out


_TINY = dict(n_heads=16, d_latent=64, d_rope=16, h_idx=4, d_idx=32, topk=32,
             act_fmt="f32", kv_fmt="f32")

WORKLOADS: dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


# -- the five measured / parity workloads -----------------------------------
_add(Workload("tiny_prefill_t256_cp4", "prefill", seed=0, seqlens=(256,),
              cp_size=4, cp_rank=1, **_TINY,
              description="one 256-token sequence, cp 4, rank 1 (64 queries);"
                          " 16 heads, latent 64 + rope 16; indexer 4x32;"
                          " top-k 32; fp32"))
_add(Workload("prefill_t8000_cp8", "prefill", seed=1, seqlens=(8000,),
              cp_size=8, cp_rank=0,
              description="one 8000-token prompt, cp 8, rank 0 (1000 queries);"
                          " 128 heads, latent 512 + rope 64; indexer 64x128;"
                          " top-k 2048; bf16"))
_add(Workload("prefill_6req_t25305_cp8", "prefill", seed=2,
              seqlens=(8000, 800, 5, 3000, 1500, 12000), cp_size=8, cp_rank=5,
              description="six requests {8000,800,5,3000,1500,12000}, cp 8,"
                          " rank 5 (3163 queries); bf16"))
_add(Workload("prefill_t65536_cp8_fp8", "prefill", seed=3, seqlens=(65536,),
              cp_size=8, cp_rank=3, kv_fmt="fp8",
              description="one 65536-token sequence, cp 8, rank 3 (8192"
                          " queries); latent KV and indexer keys e4m3fn with a"
                          " per-128-token fp32 scale; bf16 queries"))
_add(Workload("decode_32req_paged", "decode", seed=4, n_req=32, len_lo=4096,
              len_hi=65536, page_size=64,
              description="32 requests, one query each, context lengths"
                          " uniform in [4096, 65536]; 64-token pages, shuffled"
                          " page table; bf16"))

# -- smaller parity cases: several tiles, ragged tails, the oracle runs them
#    in full in seconds ------------------------------------------------------
_add(Workload("small_prefill_3req_cp4", "prefill", seed=10,
              seqlens=(1500, 611, 37), cp_size=4, cp_rank=2, topk=256,
              description="three requests, cp 4, rank 2; full model dims,"
                          " top-k 256; bf16"))
_add(Workload("small_prefill_3req_cp4_fp8", "prefill", seed=11,
              seqlens=(1500, 611, 37), cp_size=4, cp_rank=3, topk=256,
              kv_fmt="fp8", description="as above with e4m3fn KV, rank 3"))
_add(Workload("small_prefill_topk2048", "prefill", seed=12,
              seqlens=(2600,), cp_size=8, cp_rank=7, topk=2048,
              description="2600 tokens, cp 8, rank 7; top-k 2048 so that"
                          " early rows select every causal key and late rows"
                          " select a strict subset"))
_add(Workload("small_decode_paged", "decode", seed=13, n_req=5, len_lo=40,
              len_hi=3000, topk=256, page_size=64,
              description="5 requests, lengths in [40, 3000], top-k 256"))
_add(Workload("small_decode_paged_fp8", "decode", seed=14, n_req=6, len_lo=40,
              len_hi=5000, topk=256, page_size=64, kv_fmt="fp8",
              description="6 requests, lengths in [40, 5000], top-k 256; latent"
                          " KV and indexer keys e4m3fn, per-128-row scale"))
_add(Workload("long_decode_paged", "decode", seed=15, n_req=3, len_lo=66000,
              len_hi=80000, page_size=64,
              description="3 requests with contexts past 65536 keys (the"
                          " two-phase top-k); top-k 2048; bf16"))
_add(replace(WORKLOADS["tiny_prefill_t256_cp4"], name="tiny_prefill_dense",
             seed=20, topk=256,
             description="tiny prefill with top-k >= context: dense causal"))
_add(replace(WORKLOADS["small_prefill_3req_cp4"], name="small_prefill_sharp",
             seed=21, sm_scale=math.sqrt(576.0),
             description="logit scale sqrt(576) so the softmax is peaked"))
_add(Workload("tiny_prefill_bf16", "prefill", seed=22, seqlens=(300, 5, 90),
              cp_size=3, cp_rank=0, topk=64,
              description="tiny multi-request bf16 at full model dims"))
_add(Workload("small_prefill_topk777", "prefill", seed=23, seqlens=(2600, 900),
              cp_size=4, cp_rank=1, topk=777,
              description="two requests, cp 4, rank 1; top-k 777, not a"
                          " multiple of the 32-row MLA tile: a partial last"
                          " tile, and rows that select every causal key next"
                          " to rows that select a strict subset; bf16"))
_add(Workload("small_prefill_cp1", "prefill", seed=25, seqlens=(700, 300),
              cp_size=1, cp_rank=0, topk=256,
              description="no context parallelism (cp 1): the split and the"
                          " rerange are the identity; two requests; bf16"))
_add(Workload("small_prefill_cp16", "prefill", seed=26, seqlens=(1000, 37, 5),
              cp_size=16, cp_rank=15, topk=256,
              description="cp 16, last rank: a 37-token request leaves the rank"
                          " two tokens, a 5-token one none; bf16"))
_add(Workload("small_decode_splits", "decode", seed=27, n_req=4, len_lo=40,
              len_hi=3000, topk=2048, page_size=64,
              description="4 requests, lengths in [40, 3000], top-k 2048: the"
                          " MLA splits each query's 2048 slots 8 ways, and the"
                          " splits past a short context hold only -1 (empty"
                          " partials for the combine); bf16"))
_add(Workload("small_decode_splits_fp8", "decode", seed=28, n_req=4, len_lo=40,
              len_hi=3000, topk=2048, page_size=64, kv_fmt="fp8",
              description="as above with e4m3fn latent KV and indexer keys"))
_add(Workload("small_decode_topk333_fp8", "decode", seed=24, n_req=7, len_lo=40,
              len_hi=4000, topk=333, page_size=64, kv_fmt="fp8",
              description="7 requests, lengths in [40, 4000], top-k 333 (the"
                          " decode splits end off the tile grid); latent KV and"
                          " indexer keys e4m3fn"))


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; have {sorted(WORKLOADS)}")
