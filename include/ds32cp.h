/*
 * ds32cp -- one context-parallel rank's share of DeepSeek-V3.2-style sparse
 * attention on AMD Instinct MI355X (gfx950).
 *
 * The hot path, in the order the pages give it:
 *   1. cp_split_metadata   round-robin token split + per-rank metadata
 *   2. kv_rerange          rank-concatenated KV rows -> logical token order
 *   3.+4. indexer_topk     ReLU-weighted indexer scores + per-query top-k
 *   5. sparse_mla_prefill / sparse_mla_decode
 *                          latent attention over the selected rows only
 *   D. kv_cache_write      the rank keeps its own tokens' KV in the paged
 *                          cache pool for the decode steps
 *
 * Sources (cited per entry point below):
 *   [RFC]   "[RFC]: Parallel strategy for Deepseek v3.2 like models"
 *           (ROCm/ATOM issue 196): "New proposal", "Pros", "Cons" and the
 *           comment thread on the indexer and sparse MLA.
 *   [BLOG]  "[DeepSeek v3.2] 上下文并行详解" (context parallelism,
 *           explained): section 1 (summary), section 2B (split logic),
 *           section 2C (attention adaptation), section 4 part 3 (KV-cache
 *           flow: steps 1, B, C, D).
 *   [ASCEND] "Model Parallel Strategy Analysis": step 1.2 (attention core
 *           is compute-bound in prefill, memory-bound in decode) and the
 *           common-errors table (MLA's latent KV is not stored per head).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "dev" are device memory on the current HIP device;
 *   the caller owns them and keeps them alive until `stream` has finished
 *   the work.  The library allocates nothing, frees nothing and keeps no
 *   pointer after returning (sparse_mla_decode_noalloc's own scratch array,
 *   a static device array of the library, aside).
 * - Calls are asynchronous on `stream` (NULL = the default stream) and never
 *   synchronise.
 * - Arrays are dense and row-major with the shapes given; indices are
 *   int32.  bf16 arrays hold bfloat16 bit patterns; fp8 arrays hold OCP
 *   e4m3fn codes (bias 7, no infinities) with one fp32 scale per 128
 *   consecutive rows (DS_FP8_E4M3FN: value = code * scale[row / 128]) or
 *   one per row (DS_FP8_E4M3FN_ROWSCALE: value = code * scale[row]),
 *   scale >= 0.  Keys and latent rows of either fp8 format are read by
 *   sparse_mla_* and by the paged (decode) indexer; the contiguous
 *   (prefill) indexer reads the per-128-row format only.
 * - Arguments are checked on the host before any launch:
 *   DS_ERR_INVALID_ARG / DS_ERR_UNSUPPORTED / DS_ERR_WORKSPACE return
 *   without touching the device.  DS_ERR_HIP reports a failed launch; the
 *   text of every error is in ds_last_error() (per thread).
 * - Device-resident metadata (offsets, lengths, indices, page tables) is
 *   not inspected on the host; kernels clamp it so that no access leaves
 *   the buffers described by the size arguments.  Inconsistent metadata
 *   gives unspecified values, never an out-of-bounds access.
 */
#ifndef DS32CP_H
#define DS32CP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ds_dtype {
  DS_F32 = 0,
  DS_BF16 = 1,
  DS_FP8_E4M3FN = 2,          /* e4m3fn codes, one fp32 scale per 128 rows */
  DS_FP8_E4M3FN_ROWSCALE = 3  /* e4m3fn codes, one fp32 scale per row
                                 (the pools kv_cache_write_fp8 fills) */
} ds_dtype;

typedef enum ds_status {
  DS_OK = 0,
  DS_ERR_INVALID_ARG = 1,
  DS_ERR_UNSUPPORTED = 2,
  DS_ERR_WORKSPACE = 3,
  DS_ERR_HIP = 4
} ds_status;

/* Version of this interface (bumped on any change to it): 3. */
int32_t ds_abi_version(void);

/* Message describing the last error returned on the calling thread. */
const char* ds_last_error(void);

/* Number of tokens rank `cp_rank` owns under the round-robin split of
 * `num_tokens` tokens: ceil((num_tokens - cp_rank) / cp_size), 0 if
 * negative.  Host only, pure.  Returns -1 for invalid arguments.
 * [BLOG] section 1 and section 2B (token g goes to rank g mod cp_size). */
int32_t ds_cp_local_count(int64_t num_tokens, int32_t cp_size, int32_t cp_rank);

/* ---------------------------------------------------------------------
 * Step 1: round-robin split and per-rank metadata.
 * [BLOG] section 1 and 2B: token g of the flattened batch goes to rank
 * g mod cp_size; per-rank sequence lengths, batch indices and cumulative
 * offsets are recomputed after the split.  [BLOG] section 4 part 3,
 * step C: a query at position p of its request attends to positions 0..p
 * of that request (inclusive reading of the causal example there).
 *
 *   cu_seqlens [num_reqs+1] dev   cumulative offsets, cu[0] = 0,
 *                                 non-decreasing, cu[num_reqs] = num_tokens
 *   outputs, n = ds_cp_local_count(num_tokens, cp_size, cp_rank) entries
 *   unless noted (any output pointer may be NULL to skip it):
 *   local_cu   [num_reqs+1] dev   number of the rank's tokens below cu[b]
 *   batch_idx  [n] dev            request of the rank's j-th token
 *   global_idx [n] dev            its global index g_j = cp_rank + j*cp_size
 *   kv_start   [n] dev            cu[batch_idx[j]] (first KV row of the request)
 *   kv_len     [n] dev            g_j - kv_start[j] + 1 (causal key count)
 *   rows_src   [num_tokens, row_bytes] dev, or NULL: optional row gather,
 *   rows_dst   [n, row_bytes] dev        rows_dst[j] = rows_src[g_j]
 * Errors: INVALID_ARG for cp_size < 1, cp_rank outside [0, cp_size),
 * num_tokens < 0, num_reqs < 1, NULL cu_seqlens, rows_src with
 * row_bytes <= 0, or without rows_dst on a rank that owns tokens (a rank
 * with none may pass NULL).
 * ------------------------------------------------------------------- */
ds_status cp_split_metadata(const int32_t* cu_seqlens, int32_t num_reqs,
                            int32_t num_tokens, int32_t cp_size,
                            int32_t cp_rank, int32_t* local_cu,
                            int32_t* batch_idx, int32_t* global_idx,
                            int32_t* kv_start, int32_t* kv_len,
                            const void* rows_src, void* rows_dst,
                            int64_t row_bytes, hipStream_t stream);

/* Decode step metadata, the decode counterpart of cp_split_metadata: one
 * query per request; request i's query sits at position lengths[i] - 1 and
 * its own KV is already in the cache ([BLOG] section 4 part 3, step D:
 * each rank keeps its tokens' KV for the decode steps), so its causal keys
 * are positions 0 .. lengths[i] - 1 of that request.
 *   lengths [n_req] dev int32   context length of each request (< 0 read as 0)
 *   q_req, kv_start, kv_len [n_req] dev int32 outputs (any may be NULL):
 *   q_req[i] = i, kv_start[i] = 0, kv_len[i] = lengths[i]
 * Errors: INVALID_ARG for n_req < 0 or NULL lengths with n_req > 0. */
ds_status decode_metadata(const int32_t* lengths, int32_t n_req, int32_t* q_req,
                          int32_t* kv_start, int32_t* kv_len, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Contrast mode: the in-sequence split that the round-robin split replaces.
 * [BLOG] section 4 part 1: each request is cut into cp_size consecutive
 * chunks and rank r takes chunk r of every request (8000 tokens on 8
 * ranks: rank 0 tokens 0..999, rank 1 1000..1999, ...; with a second,
 * 800-token request rank 0 also takes its tokens 0..99).  Reading taken:
 * chunks of ceil(L / cp_size) tokens at token granularity (the last chunks
 * of a request may be shorter or empty).  Not on the hot path: it exists to
 * measure the per-rank imbalance the page describes.
 *
 * ds_cp_in_seq_local_count: host only, pure; cu_seqlens is a HOST array
 * [num_reqs+1].  Returns the rank's token count, or -1 for invalid
 * arguments (cp_size < 1, cp_rank outside [0, cp_size), num_reqs < 1,
 * NULL, decreasing offsets).
 *
 * cp_split_metadata_in_seq: the same outputs as cp_split_metadata, for the
 * rank's n_local tokens in request order and position order within a
 * request (n_local from ds_cp_in_seq_local_count; entries past the rank's
 * real count get batch_idx = global_idx = -1, kv_start = kv_len = 0).
 * local_cu is required (the per-token pass reads it).  The optional row
 * gather rows_dst[j] = rows_src[global_idx[j]] needs global_idx and skips
 * entries outside [0, num_tokens).
 * Errors: INVALID_ARG for cp_size < 1, cp_rank outside [0, cp_size),
 * num_tokens or n_local < 0, num_reqs < 1, NULL cu_seqlens or local_cu, a
 * row gather without global_idx, rows_dst (n_local > 0) or row_bytes > 0.
 * ------------------------------------------------------------------- */
int32_t ds_cp_in_seq_local_count(const int32_t* cu_seqlens, int32_t num_reqs,
                                 int32_t cp_size, int32_t cp_rank);

ds_status cp_split_metadata_in_seq(const int32_t* cu_seqlens, int32_t num_reqs,
                                   int32_t num_tokens, int32_t cp_size,
                                   int32_t cp_rank, int32_t n_local,
                                   int32_t* local_cu, int32_t* batch_idx,
                                   int32_t* global_idx, int32_t* kv_start,
                                   int32_t* kv_len, const void* rows_src,
                                   void* rows_dst, int64_t row_bytes,
                                   hipStream_t stream);

/* ---------------------------------------------------------------------
 * Step 2: rerange of the all-gathered KV into logical token order.
 * [BLOG] section 4 part 3, step B: after the all-gather the rows are in
 * rank-concatenated order (T0,T4,T1,T5,... for 8 tokens on 4 ranks) and
 * are put back into order T0,T1,T2,...; [BLOG] section 2C (gather and
 * rerange tuned for the round-robin mode).
 *
 *   src [cp_size*slot_rows, row_bytes] dev  rank r's j-th row at
 *                                           r*slot_rows + j; rows past a
 *                                           rank's count are never read
 *   dst [num_tokens, row_bytes] dev         dst[g] = src[(g mod cp)*slot_rows
 *                                                        + g div cp]
 * Dtype-agnostic (moves bytes).  src and dst must not overlap.
 * Errors: INVALID_ARG for cp_size < 1, num_tokens < 0, row_bytes <= 0,
 * slot_rows < ceil(num_tokens / cp_size), NULL buffers with num_tokens > 0.
 * ------------------------------------------------------------------- */
ds_status kv_rerange(const void* src, int32_t slot_rows, int32_t num_tokens,
                     int32_t cp_size, int64_t row_bytes, void* dst,
                     hipStream_t stream);

/* ---------------------------------------------------------------------
 * Steps 3 and 4: indexer scores and per-query top-k.
 * [RFC] comment thread: the indexer selects, for every query, the top-k
 * entries of its history; this per-query loop is what splitting queries
 * over ranks shortens.  [BLOG] section 2C: the indexer's KV range and the
 * top-k index transform work on the logically ordered KV.
 * Score (the pages give no formula; plainest reading):
 *     I[j, p] = sum_h w[j, h] * max(0, <q_idx[j, h, :], k_idx[row(j, p), :]>)
 * for causal positions p in [0, kv_len[j]) of query j, where
 *     prefill (page_table == NULL):  row(j, p) = kv_start[j] + p
 *     decode  (page_table != NULL):  l = kv_start[j] + p,
 *             row = page_table[q_req[j]*max_pages + l/page_size]*page_size
 *                   + l % page_size
 * Top-k: the topk largest scores of each row, ties to the lower position;
 * a row with fewer than topk causal keys selects all of them and pads with
 * -1.  Output order within a row is unspecified.
 *
 *   q_idx  [n_q, h_idx, d_idx] dev   q_dtype: DS_F32 or DS_BF16
 *   w      [n_q, h_idx] dev fp32     per-query, per-head weights
 *   k_idx  [k_rows, d_idx] dev       k_dtype: DS_F32, DS_BF16 (with bf16 or
 *                                    f32 q) or DS_FP8_E4M3FN (bf16 q)
 *   k_scale [ceil(k_rows/128)] dev fp32 for fp8 keys, else NULL
 *   kv_start, kv_len [n_q] dev       logical causal range per query
 *   q_req [n_q] dev, page_table [n_req, max_pages] dev: decode only
 *   max_kv_len                       upper bound of kv_len (host value)
 *   topk_idx [n_q, topk] dev int32   physical KV rows, -1 padded
 *   topk_score [n_q, topk] dev fp32  scores of the selected rows, or NULL
 *   ws, ws_bytes                     device workspace of at least
 *                                    indexer_topk_workspace_size(n_q, max_kv_len)
 * Supported: f32 path any h_idx <= 64, d_idx <= 128 (d_idx % 4 == 0);
 * bf16/fp8 path h_idx == 64, d_idx == 128.  topk in [1, 2048].
 * Errors: INVALID_ARG (bad sizes, NULL buffers, topk out of range),
 * UNSUPPORTED (dtype/dim combination), WORKSPACE (ws too small).
 * ------------------------------------------------------------------- */
size_t indexer_topk_workspace_size(int32_t n_q, int32_t max_kv_len);

ds_status indexer_topk(const void* q_idx, ds_dtype q_dtype, const float* w,
                       const void* k_idx, ds_dtype k_dtype,
                       const float* k_scale, int64_t k_rows,
                       const int32_t* kv_start, const int32_t* kv_len,
                       const int32_t* q_req, const int32_t* page_table,
                       int32_t n_req, int32_t page_size, int32_t max_pages,
                       int32_t n_q, int32_t h_idx, int32_t d_idx,
                       int32_t max_kv_len, int32_t topk, int32_t* topk_idx,
                       float* topk_score, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Step 3 alone: writes scores[j * score_stride + p] for p < kv_len[j]
 * (entries at or past kv_len[j] are left untouched).  Same arguments as
 * indexer_topk; score_stride >= max_kv_len. */
ds_status indexer_scores(const void* q_idx, ds_dtype q_dtype, const float* w,
                         const void* k_idx, ds_dtype k_dtype,
                         const float* k_scale, int64_t k_rows,
                         const int32_t* kv_start, const int32_t* kv_len,
                         const int32_t* q_req, const int32_t* page_table,
                         int32_t n_req, int32_t page_size, int32_t max_pages,
                         int32_t n_q, int32_t h_idx, int32_t d_idx,
                         int32_t max_kv_len, float* scores,
                         int64_t score_stride, hipStream_t stream);

/* Step 4 alone: top-k of precomputed score rows (layout as written by
 * indexer_scores), mapped to physical rows as described above. */
ds_status topk_select(const float* scores, int64_t score_stride,
                      const int32_t* kv_start, const int32_t* kv_len,
                      const int32_t* q_req, const int32_t* page_table,
                      int32_t n_req, int32_t page_size, int32_t max_pages,
                      int64_t k_rows, int32_t n_q, int32_t max_kv_len,
                      int32_t topk, int32_t* topk_idx, float* topk_score,
                      hipStream_t stream);

/* ---------------------------------------------------------------------
 * Step 5: sparse latent attention (MLA) over the selected rows.
 * [RFC] comment thread: each query attends only to its top-k KV entries
 * instead of to all KV; "Pros": every rank keeps all heads of MLA, which
 * gives a high-intensity contraction.  [ASCEND] common-errors table: the
 * latent KV is one vector per token shared by all heads.  Reading taken
 * (the pages give no formula): absorbed latent form,
 *     logit[h, s] = sm_scale * <q[j, h, :], kv[s, :]>   (d_latent + d_rope)
 *     out[j, h, :] = sum_s softmax_s(logit[h, :]) * kv[s, :d_latent]
 *     lse[j, h]    = log sum_s exp(logit[h, s])          (natural log)
 * over s in {topk_idx[j, i] : 0 <= topk_idx[j, i] < kv_rows}; entries of
 * -1 (or out of range) are skipped; a row with no entries gives out = 0,
 * lse = -inf.  Rope parts are already applied to q and kv.
 *
 *   q   [n_q, n_heads, d_latent + d_rope] dev   q_dtype
 *   kv  [kv_rows, d_latent + d_rope] dev        kv_dtype
 *   kv_scale [ceil(kv_rows/128)] dev fp32       fp8 only, else NULL
 *   topk_idx [n_q, topk] dev int32              physical rows
 *   out [n_q, n_heads, d_latent] dev            out_dtype (DS_F32/DS_BF16)
 *   lse [n_q, n_heads] dev fp32, or NULL
 * Supported: all-f32 path with n_heads <= 128, d_latent + d_rope <= 640;
 * bf16 q with bf16 or fp8 kv: n_heads 32, 64 or 128 (DS_ERR_UNSUPPORTED
 * otherwise), d_latent == 512, d_rope == 64.  topk in [1, 2048].  sm_scale must be
 * positive and finite (DS_ERR_INVALID_ARG otherwise).
 * fp8 kv (prefill): the rows are first widened once per call into the
 * caller's workspace as bf16 values code * scale (round to nearest even;
 * relative error <= 2^-9 per element), and the bf16 path runs on them.
 * ws [>= sparse_mla_prefill_workspace_size(kv_rows, kv_dtype) bytes] dev,
 * 256-byte aligned; NULL is accepted when that size is 0 (bf16/f32 kv).
 * The decode variant splits each query's selected rows across workgroups
 * and merges the partial results by their log-sum-exp; it needs
 * ws_bytes >= sparse_mla_workspace_size(...).  The partial outputs are
 * held in bf16 (their maxima and sums in fp32), so its results match the
 * prefill variant's up to one bf16 rounding of each partial (relative
 * error <= 2^-9) (fp8 kv: it uses the codes exactly).
 * ------------------------------------------------------------------- */
size_t sparse_mla_prefill_workspace_size(int64_t kv_rows, ds_dtype kv_dtype);

ds_status sparse_mla_prefill(const void* q, ds_dtype q_dtype, const void* kv,
                             ds_dtype kv_dtype, const float* kv_scale,
                             int64_t kv_rows, const int32_t* topk_idx,
                             int32_t n_q, int32_t n_heads, int32_t d_latent,
                             int32_t d_rope, int32_t topk, float sm_scale,
                             void* out, ds_dtype out_dtype, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);

size_t sparse_mla_workspace_size(int32_t n_q, int32_t n_heads,
                                 int32_t d_latent, int32_t topk);

ds_status sparse_mla_decode(const void* q, ds_dtype q_dtype, const void* kv,
                            ds_dtype kv_dtype, const float* kv_scale,
                            int64_t kv_rows, const int32_t* topk_idx,
                            int32_t n_q, int32_t n_heads, int32_t d_latent,
                            int32_t d_rope, int32_t topk, float sm_scale,
                            void* out, ds_dtype out_dtype, float* lse,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------
 * The dense projections on either side of the path.  [ASCEND] step 3.1
 * (MLA's q_down / q_up / kv_down / kv_up (K, V) / o_proj projections);
 * [RFC] "Problem with tp" (the indexer's wq_b and w_k, run by every rank on
 * every token under tensor parallelism; here each rank runs them on its
 * own tokens).  With the latent attention the K up-projection folds into
 * the queries (q_latent[h] = q_nope[h] . W_UK[h]) and the V up-projection
 * into the output (o[h] = O_latent[h] . W_UV[h]); both are batched over
 * the heads.  One batched GEMM serves all of them:
 *     C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]       (fp32 accumulation)
 *   A  bf16, row m of batch b at A + b*stride_a + m*lda (K values, contiguous)
 *   B  bf16, row n of batch b at B + b*stride_b + n*ldb (weights as [out, in])
 *   C  bf16 (round to nearest even) or f32, C + b*stride_c + m*ldc + n
 *   strides and leading dimensions in elements; per-head slices of wider
 *   rows are addressed in place (e.g. the latent part of a 576-wide row)
 *   ws  split-K partials, gemm_bf16_nt_workspace_size() bytes (0: none)
 * Supported: K a multiple of 64, N a multiple of 128, A and B 16-byte
 * aligned with lda, ldb, stride_a, stride_b multiples of 8.  C must not
 * overlap A or B.
 * Errors: INVALID_ARG (negative sizes, NULL operands, lda < K, ldb < K,
 * ldc < N, misalignment), UNSUPPORTED (K, N or C dtype), WORKSPACE.
 * ------------------------------------------------------------------- */
size_t gemm_bf16_nt_workspace_size(int32_t M, int32_t N, int32_t K, int32_t batch);

ds_status gemm_bf16_nt(const void* A, int64_t lda, int64_t stride_a, const void* B,
                       int64_t ldb, int64_t stride_b, void* C, ds_dtype c_dtype,
                       int64_t ldc, int64_t stride_c, int32_t M, int32_t N, int32_t K,
                       int32_t batch, void* ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of sparse_mla_decode, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * and results as sparse_mla_decode without ws/ws_bytes: the split partials
 * live in a library-owned device array of
 * sparse_mla_decode_noalloc_scratch_bytes() bytes (32 MiB), one per GPU,
 * held until the process ends.  When the default split count's partials
 * (n_q * splits * n_heads * 1 KB, plus their maxima and sums) would not fit,
 * the call takes the largest split count that fits, down to one split,
 * which needs no scratch; the results then differ from sparse_mla_decode's
 * only by the bf16 rounding of fewer partials.  The call allocates nothing
 * and never fails for size.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race and give unspecified results; the array keeps the last
 * call's contents, and nothing in it needs to start at zero.
 * Errors: as sparse_mla_decode; DS_ERR_HIP if the array's device address
 * cannot be obtained. */
size_t sparse_mla_decode_noalloc_scratch_bytes(void);

ds_status sparse_mla_decode_noalloc(const void* q, ds_dtype q_dtype, const void* kv,
                                    ds_dtype kv_dtype, const float* kv_scale,
                                    int64_t kv_rows, const int32_t* topk_idx,
                                    int32_t n_q, int32_t n_heads, int32_t d_latent,
                                    int32_t d_rope, int32_t topk, float sm_scale,
                                    void* out, ds_dtype out_dtype, float* lse,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------
 * Step D: the rank keeps its own tokens' KV in the paged cache pool.
 * [BLOG] section 4 part 3, step D: after attention the gathered global KV
 * is dropped, and each rank keeps only the KV of the tokens it owns (rank 1
 * keeps K1, K5 of the 8-token example) in the device cache pool, for the
 * decode steps.
 *
 *   rows       [n_local, row_bytes] dev   the rank's own rows in local order
 *                                         (cp_split_metadata's rows_dst)
 *   batch_idx  [n_local] dev int32        request of each local row
 *   local_cu   [n_req + 1] dev int32      first local row of each request
 *                                         (both from cp_split_metadata)
 *   page_table [n_req, max_pages] dev int32  page ids of each request's
 *                                         cache; -1 = not mapped
 *   pool       [pool_rows, row_bytes] dev written in place
 * Local row j, of request b = batch_idx[j] and cache position
 * p = j - local_cu[b], is copied to pool row
 * page_table[b][p / page_size] * page_size + p % page_size: the mapping the
 * decode calls read through.  A row is not written when b is outside
 * [0, n_req), p < 0, p / page_size >= max_pages, the page id is negative or
 * the pool row is >= pool_rows; nothing else in the pool changes.
 * Dtype-agnostic (moves bytes: the pool keeps the rows' storage format).
 * rows and pool must not overlap.  If the table maps two positions to one
 * pool row, either row may be kept.
 * Errors: INVALID_ARG for n_local, n_req, max_pages or pool_rows < 0,
 * page_size < 1, row_bytes <= 0, NULL buffers that are needed (n_local > 0),
 * overlapping rows and pool.
 * ------------------------------------------------------------------- */
ds_status kv_cache_write(const void* rows, int32_t n_local, int64_t row_bytes,
                         const int32_t* batch_idx, const int32_t* local_cu, int32_t n_req,
                         const int32_t* page_table, int32_t max_pages, int32_t page_size,
                         void* pool, int64_t pool_rows, hipStream_t stream);

/* Step D with fp8 encoding: [BLOG] section 1 (the round-robin split lifts
 * the old split's "no FP8 KV cache" limit) and section 4 part 3 step D.
 * Each local row (bf16, row_elems values) is encoded on its own and stored
 * where kv_cache_write stores it: pool_codes[phys] gets the e4m3fn codes
 * and pool_scale[phys] the row's scale, so the pool is read back as
 * DS_FP8_E4M3FN_ROWSCALE.  Encoding (the pages give none): scale = row
 * amax / 448 (fp32, correctly rounded), code = e4m3fn nearest to
 * x / scale, ties to even, with x / scale clamped to [-448, 448]; an
 * all-zero row stores scale 0 and zero codes.  A scale per row keeps rows
 * of different requests, written at different times, apart: no write
 * re-encodes a row it does not own.  Rows must be finite.
 *   rows        [n_local, row_elems] dev bf16 (rows_dtype DS_BF16), 8-byte aligned
 *   batch_idx, local_cu, page_table, max_pages, page_size: as kv_cache_write
 *   pool_codes  [pool_rows, row_elems] dev uint8, 4-byte aligned, in place
 *   pool_scale  [pool_rows] dev fp32, in place
 * Supported: row_elems a multiple of 4 in [4, 1024] (576 latent, 128
 * indexer-key values).  Errors: UNSUPPORTED for other row sizes or row
 * dtypes; INVALID_ARG as kv_cache_write, and for misaligned rows/codes. */
ds_status kv_cache_write_fp8(const void* rows, ds_dtype rows_dtype, int32_t n_local,
                             int32_t row_elems, const int32_t* batch_idx,
                             const int32_t* local_cu, int32_t n_req,
                             const int32_t* page_table, int32_t max_pages,
                             int32_t page_size, uint8_t* pool_codes, float* pool_scale,
                             int64_t pool_rows, hipStream_t stream);


#ifdef __cplusplus
}
#endif

#endif /* DS32CP_H */
