"""MI355X-native round-robin context-parallel sparse attention (DeepSeek-V3.2 style).

One context-parallel rank's share of the attention hot path, as hand-written
HIP kernels for gfx950 behind the C ABI of ``include/ds32cp.h``:

1. ``cp_split_metadata`` -- round-robin token split + per-rank metadata
2. ``kv_rerange``        -- rank-concatenated KV rows -> logical order
3. + 4. ``indexer_topk`` -- ReLU-weighted indexer scores + per-query top-k
5. ``sparse_mla_prefill`` / ``sparse_mla_decode`` -- latent attention over
   the selected rows

This package is the thin ctypes binding (argument marshalling only; torch
supplies device memory and streams).  Importing it loads ``libds32cp.so``
and fails loudly if the library has not been built.
"""

from ._lib import (  # noqa: F401
    DS32CPError, DS_BF16, DS_F32, DS_FP8_E4M3FN, DS_FP8_E4M3FN_ROWSCALE, LIB_PATH, abi_version,
    cp_in_seq_local_count, cp_local_count, cp_split_metadata, cp_split_metadata_in_seq,
    decode_metadata, gemm_bf16_nt, gemm_bf16_nt_workspace_size, indexer_scores,
    indexer_topk, indexer_topk_workspace_size, kv_cache_write, kv_cache_write_fp8, kv_rerange,
    sparse_mla_decode,
    sparse_mla_decode_noalloc,
    sparse_mla_prefill, sparse_mla_prefill_workspace_size, sparse_mla_workspace_size, topk_select,
)
