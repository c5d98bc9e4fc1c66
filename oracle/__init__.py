"""CPU oracle for round-robin context-parallel sparse attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy (fp64) restatement of what the hot path computes.  Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library under
``deepseek_v3_context_amd/`` and imports nothing from it.

Sources (the pages this restates):

* "[RFC]: Parallel strategy for Deepseek v3.2 like models" (ROCm/ATOM
  issue 196) -- the proposal to split attention over the token dimension,
  its Pros/Cons lists, and the comment thread describing the indexer and
  sparse MLA.
* "[DeepSeek v3.2] 上下文并行详解" (context parallelism, explained) --
  section 1 (summary of the round-robin mode), section 2B (split logic),
  section 2C (attention-layer adaptation), section 4 part 1 (contiguous
  split) and section 4 part 3 (the KV-cache flow: scatter, gather +
  rerange, attention, retention).

Modules:

* :mod:`oracle.round_robin_cp` -- token ownership, per-rank metadata, the
  row split, the rank-concatenated buffer and the rerange (plain integer
  definitions).
* :mod:`oracle.sparse_attention` -- storage-format decoding (bf16, OCP
  e4m3fn), indexer scores, top-k selection, sparse latent attention (fp64).
* :mod:`oracle.pipeline` -- the steps chained for chosen query rows.
* :mod:`oracle.kv_cache` -- the rank keeping its own tokens' KV in the
  paged cache pool after attention (section 4 part 3, step D), as given or
  encoded as fp8 with a scale per row.
* :mod:`oracle.projections` -- the dense projections on either side of the
  path (the indexer's and MLA's linear layers, the latent-form absorption).

Parity status of each function is stated in its docstring; every function
here is pinned by ``tests/test_oracle_*.py`` against values the pages print,
closed forms, library routines on special cases, or brute force.
"""

from . import round_robin_cp, sparse_attention, pipeline, kv_cache, projections  # noqa: F401
