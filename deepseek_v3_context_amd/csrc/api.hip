// Host side of the C ABI declared in include/ds32cp.h: argument checks
// (before any launch), workspace sizing and dispatch to the kernels.
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <string>

#include "common.h"

namespace ds32cp {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

ds_status fail(ds_status code, const std::string& msg) {
  set_error(msg);
  return code;
}

ds_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DS_OK;
}

int32_t device_cu_count() {
  static std::atomic<int32_t> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int32_t c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

static bool is_act_dtype(ds_dtype d) { return d == DS_F32 || d == DS_BF16; }

// Library-owned scratch of the allocation-free decode entry point: the
// split partials of sparse_mla_decode_noalloc.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code the array's
// name is not a device address: its address on a device comes from
// hipGetSymbolAddress (once per device, with that device current).
constexpr size_t kNoAllocScratchBytes = 32u << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static ds_status scratch_ptr(void** out) {
  static std::once_flag once[kMaxDevices];
  static void* ptr[kMaxDevices] = {};
  static hipError_t err[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DS_ERR_HIP, "sparse_mla_decode_noalloc: no current HIP device");
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    ptr[dev] = err[dev] == hipSuccess ? p : nullptr;
  });
  if (ptr[dev] == nullptr)
    return fail(DS_ERR_HIP, std::string("sparse_mla_decode_noalloc: hipGetSymbolAddress: ") +
                                hipGetErrorString(err[dev]));
  *out = ptr[dev];
  return DS_OK;
}

}  // namespace ds32cp

using namespace ds32cp;

#define DS_REQUIRE(cond, code, msg) \
  do {                              \
    if (!(cond)) return fail((code), (msg)); \
  } while (0)

extern "C" {

int32_t ds_abi_version(void) { return 3; }

const char* ds_last_error(void) { return g_last_error.c_str(); }

int32_t ds_cp_local_count(int64_t num_tokens, int32_t cp_size, int32_t cp_rank) {
  if (cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size || num_tokens < 0) return -1;
  if (num_tokens <= cp_rank) return 0;
  const int64_t n = (num_tokens - cp_rank + cp_size - 1) / cp_size;
  return n > INT32_MAX ? -1 : static_cast<int32_t>(n);
}

ds_status cp_split_metadata(const int32_t* cu_seqlens, int32_t num_reqs,
                            int32_t num_tokens, int32_t cp_size, int32_t cp_rank,
                            int32_t* local_cu, int32_t* batch_idx,
                            int32_t* global_idx, int32_t* kv_start,
                            int32_t* kv_len, const void* rows_src, void* rows_dst,
                            int64_t row_bytes, hipStream_t stream) {
  DS_REQUIRE(cp_size >= 1, DS_ERR_INVALID_ARG, "cp_split_metadata: cp_size must be >= 1");
  DS_REQUIRE(cp_rank >= 0 && cp_rank < cp_size, DS_ERR_INVALID_ARG,
             "cp_split_metadata: cp_rank outside [0, cp_size)");
  DS_REQUIRE(num_tokens >= 0, DS_ERR_INVALID_ARG, "cp_split_metadata: num_tokens < 0");
  DS_REQUIRE(num_reqs >= 1, DS_ERR_INVALID_ARG, "cp_split_metadata: num_reqs must be >= 1");
  DS_REQUIRE(cu_seqlens != nullptr, DS_ERR_INVALID_ARG, "cp_split_metadata: cu_seqlens is NULL");
  const int32_t n = ds_cp_local_count(num_tokens, cp_size, cp_rank);
  // a rank that owns no token gathers no row: its (empty) rows_dst may be NULL
  DS_REQUIRE(rows_src == nullptr || (row_bytes > 0 && (rows_dst != nullptr || n == 0)),
             DS_ERR_INVALID_ARG,
             "cp_split_metadata: row gather needs rows_dst and row_bytes > 0");
  ds_status st = launch_split_metadata(cu_seqlens, num_reqs, num_tokens, cp_size, cp_rank,
                                       n, local_cu, batch_idx, global_idx, kv_start,
                                       kv_len, stream);
  if (st != DS_OK || rows_src == nullptr) return st;
  return launch_row_gather_rr(rows_src, rows_dst, n, cp_size, cp_rank, row_bytes, stream);
}

int32_t ds_cp_in_seq_local_count(const int32_t* cu_seqlens, int32_t num_reqs, int32_t cp_size,
                                 int32_t cp_rank) {
  if (cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size || num_reqs < 1 || cu_seqlens == nullptr)
    return -1;
  int64_t n = 0;
  for (int32_t b = 0; b < num_reqs; ++b) {
    const int64_t len = static_cast<int64_t>(cu_seqlens[b + 1]) - cu_seqlens[b];
    if (len < 0) return -1;
    const int64_t c = (len + cp_size - 1) / cp_size;
    const int64_t left = len - cp_rank * c;
    n += left <= 0 ? 0 : (left < c ? left : c);
  }
  return n > INT32_MAX ? -1 : static_cast<int32_t>(n);
}

ds_status cp_split_metadata_in_seq(const int32_t* cu_seqlens, int32_t num_reqs,
                                   int32_t num_tokens, int32_t cp_size, int32_t cp_rank,
                                   int32_t n_local, int32_t* local_cu, int32_t* batch_idx,
                                   int32_t* global_idx, int32_t* kv_start, int32_t* kv_len,
                                   const void* rows_src, void* rows_dst, int64_t row_bytes,
                                   hipStream_t stream) {
  const char* f = "cp_split_metadata_in_seq";
  DS_REQUIRE(cp_size >= 1, DS_ERR_INVALID_ARG, std::string(f) + ": cp_size must be >= 1");
  DS_REQUIRE(cp_rank >= 0 && cp_rank < cp_size, DS_ERR_INVALID_ARG,
             std::string(f) + ": cp_rank outside [0, cp_size)");
  DS_REQUIRE(num_tokens >= 0 && n_local >= 0, DS_ERR_INVALID_ARG,
             std::string(f) + ": num_tokens and n_local must be >= 0");
  DS_REQUIRE(num_reqs >= 1, DS_ERR_INVALID_ARG, std::string(f) + ": num_reqs must be >= 1");
  DS_REQUIRE(cu_seqlens != nullptr && local_cu != nullptr, DS_ERR_INVALID_ARG,
             std::string(f) + ": cu_seqlens and local_cu are required");
  DS_REQUIRE(rows_src == nullptr ||
                 (row_bytes > 0 && ((global_idx != nullptr && rows_dst != nullptr) || n_local == 0)),
             DS_ERR_INVALID_ARG,
             std::string(f) + ": row gather needs global_idx, rows_dst and row_bytes > 0");
  return launch_in_seq_split(cu_seqlens, num_reqs, num_tokens, cp_size, cp_rank, n_local,
                             local_cu, batch_idx, global_idx, kv_start, kv_len, rows_src,
                             rows_dst, row_bytes, stream);
}

ds_status decode_metadata(const int32_t* lengths, int32_t n_req, int32_t* q_req,
                          int32_t* kv_start, int32_t* kv_len, hipStream_t stream) {
  DS_REQUIRE(n_req >= 0, DS_ERR_INVALID_ARG, "decode_metadata: n_req < 0");
  DS_REQUIRE(n_req == 0 || lengths != nullptr, DS_ERR_INVALID_ARG, "decode_metadata: NULL lengths");
  return launch_decode_metadata(lengths, n_req, q_req, kv_start, kv_len, stream);
}

ds_status kv_rerange(const void* src, int32_t slot_rows, int32_t num_tokens,
                     int32_t cp_size, int64_t row_bytes, void* dst,
                     hipStream_t stream) {
  DS_REQUIRE(cp_size >= 1, DS_ERR_INVALID_ARG, "kv_rerange: cp_size must be >= 1");
  DS_REQUIRE(num_tokens >= 0, DS_ERR_INVALID_ARG, "kv_rerange: num_tokens < 0");
  DS_REQUIRE(row_bytes > 0, DS_ERR_INVALID_ARG, "kv_rerange: row_bytes must be > 0");
  DS_REQUIRE(static_cast<int64_t>(slot_rows) * cp_size >= num_tokens && slot_rows >= 0,
             DS_ERR_INVALID_ARG, "kv_rerange: slot_rows < ceil(num_tokens / cp_size)");
  DS_REQUIRE(num_tokens == 0 || (src != nullptr && dst != nullptr), DS_ERR_INVALID_ARG,
             "kv_rerange: NULL buffer");
  if (num_tokens > 0) {
    const char* s0 = static_cast<const char*>(src);
    const char* d0 = static_cast<const char*>(dst);
    const int64_t sb = static_cast<int64_t>(slot_rows) * cp_size * row_bytes;
    const int64_t db = static_cast<int64_t>(num_tokens) * row_bytes;
    DS_REQUIRE(s0 + sb <= d0 || d0 + db <= s0, DS_ERR_INVALID_ARG,
               "kv_rerange: src and dst overlap");
  }
  return launch_rerange(src, dst, num_tokens, cp_size, slot_rows, row_bytes, stream);
}

ds_status kv_cache_write(const void* rows, int32_t n_local, int64_t row_bytes,
                         const int32_t* batch_idx, const int32_t* local_cu, int32_t n_req,
                         const int32_t* page_table, int32_t max_pages, int32_t page_size,
                         void* pool, int64_t pool_rows, hipStream_t stream) {
  DS_REQUIRE(n_local >= 0 && n_req >= 0 && max_pages >= 0 && pool_rows >= 0,
             DS_ERR_INVALID_ARG, "kv_cache_write: negative size");
  DS_REQUIRE(page_size >= 1, DS_ERR_INVALID_ARG, "kv_cache_write: page_size must be >= 1");
  DS_REQUIRE(row_bytes > 0, DS_ERR_INVALID_ARG, "kv_cache_write: row_bytes must be > 0");
  if (n_local == 0) return DS_OK;
  DS_REQUIRE(rows != nullptr && batch_idx != nullptr && local_cu != nullptr &&
                 (pool != nullptr || pool_rows == 0) &&
                 (page_table != nullptr || static_cast<int64_t>(n_req) * max_pages == 0),
             DS_ERR_INVALID_ARG, "kv_cache_write: NULL buffer");
  if (pool_rows > 0) {
    const char* s0 = static_cast<const char*>(rows);
    const char* d0 = static_cast<const char*>(pool);
    const int64_t sb = static_cast<int64_t>(n_local) * row_bytes;
    const int64_t db = pool_rows * row_bytes;
    DS_REQUIRE(s0 + sb <= d0 || d0 + db <= s0, DS_ERR_INVALID_ARG,
               "kv_cache_write: rows and pool overlap");
  }
  if (pool_rows == 0 || static_cast<int64_t>(n_req) * max_pages == 0) return DS_OK;   // nothing maps
  return launch_kv_cache_write(rows, n_local, row_bytes, batch_idx, local_cu, n_req,
                               page_table, max_pages, page_size, pool, pool_rows, stream);
}

ds_status kv_cache_write_fp8(const void* rows, ds_dtype rows_dtype, int32_t n_local,
                             int32_t row_elems, const int32_t* batch_idx, const int32_t* local_cu,
                             int32_t n_req, const int32_t* page_table, int32_t max_pages,
                             int32_t page_size, uint8_t* pool_codes, float* pool_scale,
                             int64_t pool_rows, hipStream_t stream) {
  const char* f = "kv_cache_write_fp8";
  DS_REQUIRE(rows_dtype == DS_BF16, DS_ERR_UNSUPPORTED, std::string(f) + ": rows must be bf16");
  DS_REQUIRE(n_local >= 0 && n_req >= 0 && max_pages >= 0 && pool_rows >= 0,
             DS_ERR_INVALID_ARG, std::string(f) + ": negative size");
  DS_REQUIRE(page_size >= 1, DS_ERR_INVALID_ARG, std::string(f) + ": page_size must be >= 1");
  DS_REQUIRE(row_elems >= 1 && row_elems <= kCacheFp8MaxElems && row_elems % 4 == 0,
             DS_ERR_UNSUPPORTED,
             std::string(f) + ": row_elems must be a multiple of 4 in [4, 1024]");
  if (n_local == 0) return DS_OK;
  DS_REQUIRE(rows != nullptr && batch_idx != nullptr && local_cu != nullptr &&
                 ((pool_codes != nullptr && pool_scale != nullptr) || pool_rows == 0) &&
                 (page_table != nullptr || static_cast<int64_t>(n_req) * max_pages == 0),
             DS_ERR_INVALID_ARG, std::string(f) + ": NULL buffer");
  DS_REQUIRE((reinterpret_cast<uintptr_t>(rows) & 7) == 0 &&
                 (reinterpret_cast<uintptr_t>(pool_codes) & 3) == 0,
             DS_ERR_INVALID_ARG, std::string(f) + ": rows must be 8-byte and codes 4-byte aligned");
  if (pool_rows == 0 || static_cast<int64_t>(n_req) * max_pages == 0) return DS_OK;   // nothing maps
  return launch_kv_cache_write_fp8(rows, n_local, row_elems, batch_idx, local_cu, n_req,
                                   page_table, max_pages, page_size, pool_codes, pool_scale,
                                   pool_rows, stream);
}

static ds_status check_indexer(const char* fn, const IndexerArgs& a) {
  const std::string f(fn);
  DS_REQUIRE(a.n_q >= 0 && a.max_kv_len >= 0 && a.k_rows >= 0, DS_ERR_INVALID_ARG,
             f + ": negative size");
  DS_REQUIRE(a.h_idx >= 1 && a.d_idx >= 1, DS_ERR_INVALID_ARG, f + ": h_idx/d_idx must be >= 1");
  if (a.n_q > 0) {
    DS_REQUIRE(a.q_idx && a.w && a.kv_start && a.kv_len, DS_ERR_INVALID_ARG,
               f + ": NULL query/weight/metadata pointer");
    DS_REQUIRE(a.k_rows == 0 || a.k_idx, DS_ERR_INVALID_ARG, f + ": NULL key pointer");
  }
  DS_REQUIRE(is_act_dtype(a.q_dtype), DS_ERR_UNSUPPORTED, f + ": q_idx must be f32 or bf16");
  if (a.page_table != nullptr) {
    DS_REQUIRE(a.q_req != nullptr, DS_ERR_INVALID_ARG, f + ": paged keys need q_req");
    DS_REQUIRE(a.page_size >= 1 && a.max_pages >= 1 && a.n_req >= 1, DS_ERR_INVALID_ARG,
               f + ": page_size, max_pages and n_req must be >= 1");
  }
  if (a.q_dtype == DS_F32) {
    DS_REQUIRE(a.k_dtype == DS_F32 || a.k_dtype == DS_BF16, DS_ERR_UNSUPPORTED,
               f + ": f32 queries need f32 or bf16 keys");
    DS_REQUIRE(a.h_idx <= 64 && a.d_idx <= 128, DS_ERR_UNSUPPORTED,
               f + ": f32 path supports h_idx <= 64, d_idx <= 128");
  } else {
    DS_REQUIRE(a.k_dtype == DS_BF16 || a.k_dtype == DS_FP8_E4M3FN ||
                   a.k_dtype == DS_FP8_E4M3FN_ROWSCALE,
               DS_ERR_UNSUPPORTED, f + ": bf16 queries need bf16 or fp8 keys");
    DS_REQUIRE(a.k_dtype != DS_FP8_E4M3FN_ROWSCALE || a.page_table != nullptr,
               DS_ERR_UNSUPPORTED, f + ": fp8 keys with a scale per row are read from a paged pool");
    DS_REQUIRE(a.h_idx == 64 && a.d_idx == 128, DS_ERR_UNSUPPORTED,
               f + ": bf16 path supports h_idx == 64, d_idx == 128");
  }
  if (a.k_dtype == DS_FP8_E4M3FN || a.k_dtype == DS_FP8_E4M3FN_ROWSCALE)
    DS_REQUIRE(a.k_scale != nullptr, DS_ERR_INVALID_ARG, f + ": fp8 keys need k_scale");
  return DS_OK;
}

// The kernels see one fp8 format; the scale granularity goes in a shift.
static void normalize_fp8(IndexerArgs& a) {
  if (a.k_dtype == DS_FP8_E4M3FN_ROWSCALE) {
    a.k_dtype = DS_FP8_E4M3FN;
    a.k_scale_shift = 0;
  }
}
static void normalize_fp8(MlaArgs& a) {
  if (a.kv_dtype == DS_FP8_E4M3FN_ROWSCALE) {
    a.kv_dtype = DS_FP8_E4M3FN;
    a.scale_shift = 0;
  }
}

size_t indexer_topk_workspace_size(int32_t n_q, int32_t max_kv_len) {
  if (n_q <= 0 || max_kv_len <= 0) return 256;
  size_t bytes = sizeof(float) * static_cast<size_t>(n_q) * static_cast<size_t>(round_up(max_kv_len, 64));
  if (topk_two_phase(n_q, max_kv_len)) bytes += topk_two_phase_bytes(n_q, max_kv_len);
  return bytes;
}

ds_status indexer_scores(const void* q_idx, ds_dtype q_dtype, const float* w,
                         const void* k_idx, ds_dtype k_dtype, const float* k_scale,
                         int64_t k_rows, const int32_t* kv_start, const int32_t* kv_len,
                         const int32_t* q_req, const int32_t* page_table, int32_t n_req,
                         int32_t page_size, int32_t max_pages, int32_t n_q, int32_t h_idx,
                         int32_t d_idx, int32_t max_kv_len, float* scores,
                         int64_t score_stride, hipStream_t stream) {
  IndexerArgs a{q_idx, q_dtype, w, k_idx, k_dtype, k_scale, k_rows, kv_start, kv_len,
                q_req, page_table, n_req, page_size, max_pages, n_q, h_idx, d_idx,
                max_kv_len, scores, score_stride};
  ds_status st = check_indexer("indexer_scores", a);
  if (st != DS_OK) return st;
  DS_REQUIRE(score_stride >= max_kv_len, DS_ERR_INVALID_ARG,
             "indexer_scores: score_stride < max_kv_len");
  DS_REQUIRE(n_q == 0 || scores != nullptr, DS_ERR_INVALID_ARG, "indexer_scores: NULL scores");
  normalize_fp8(a);
  return launch_indexer_scores(a, stream);
}

static ds_status check_topk(const char* fn, int32_t n_q, int32_t topk, const int32_t* idx,
                            const int32_t* kv_start, const int32_t* kv_len,
                            const int32_t* q_req, const int32_t* page_table,
                            int32_t n_req, int32_t page_size, int32_t max_pages) {
  const std::string f(fn);
  DS_REQUIRE(topk >= 1 && topk <= 2048, DS_ERR_INVALID_ARG, f + ": topk must be in [1, 2048]");
  DS_REQUIRE(n_q == 0 || (idx && kv_start && kv_len), DS_ERR_INVALID_ARG,
             f + ": NULL topk_idx or metadata");
  if (page_table != nullptr)
    DS_REQUIRE(q_req != nullptr && page_size >= 1 && max_pages >= 1 && n_req >= 1,
               DS_ERR_INVALID_ARG, f + ": bad paging arguments");
  return DS_OK;
}

ds_status topk_select(const float* scores, int64_t score_stride, const int32_t* kv_start,
                      const int32_t* kv_len, const int32_t* q_req,
                      const int32_t* page_table, int32_t n_req, int32_t page_size,
                      int32_t max_pages, int64_t k_rows, int32_t n_q, int32_t max_kv_len,
                      int32_t topk, int32_t* topk_idx, float* topk_score,
                      hipStream_t stream) {
  DS_REQUIRE(n_q >= 0 && max_kv_len >= 0 && k_rows >= 0, DS_ERR_INVALID_ARG,
             "topk_select: negative size");
  DS_REQUIRE(score_stride >= max_kv_len, DS_ERR_INVALID_ARG, "topk_select: score_stride < max_kv_len");
  DS_REQUIRE(n_q == 0 || scores != nullptr, DS_ERR_INVALID_ARG, "topk_select: NULL scores");
  ds_status st = check_topk("topk_select", n_q, topk, topk_idx, kv_start, kv_len, q_req,
                            page_table, n_req, page_size, max_pages);
  if (st != DS_OK) return st;
  TopkArgs t{scores, score_stride, kv_start, kv_len, q_req, page_table, n_req, page_size,
             max_pages, k_rows, n_q, max_kv_len, topk, topk_idx, topk_score};
  return launch_topk(t, stream);
}

ds_status indexer_topk(const void* q_idx, ds_dtype q_dtype, const float* w,
                       const void* k_idx, ds_dtype k_dtype, const float* k_scale,
                       int64_t k_rows, const int32_t* kv_start, const int32_t* kv_len,
                       const int32_t* q_req, const int32_t* page_table, int32_t n_req,
                       int32_t page_size, int32_t max_pages, int32_t n_q, int32_t h_idx,
                       int32_t d_idx, int32_t max_kv_len, int32_t topk,
                       int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  const int64_t stride = round_up(max_kv_len > 0 ? max_kv_len : 1, 64);
  IndexerArgs a{q_idx, q_dtype, w, k_idx, k_dtype, k_scale, k_rows, kv_start, kv_len,
                q_req, page_table, n_req, page_size, max_pages, n_q, h_idx, d_idx,
                max_kv_len, static_cast<float*>(ws), stride};
  ds_status st = check_indexer("indexer_topk", a);
  if (st != DS_OK) return st;
  st = check_topk("indexer_topk", n_q, topk, topk_idx, kv_start, kv_len, q_req, page_table,
                  n_req, page_size, max_pages);
  if (st != DS_OK) return st;
  DS_REQUIRE(ws != nullptr && ws_bytes >= indexer_topk_workspace_size(n_q, max_kv_len),
             DS_ERR_WORKSPACE, "indexer_topk: workspace smaller than indexer_topk_workspace_size()");
  normalize_fp8(a);
  st = launch_indexer_scores(a, stream);
  if (st != DS_OK) return st;
  TopkArgs t{static_cast<const float*>(ws), stride, kv_start, kv_len, q_req, page_table,
             n_req, page_size, max_pages, k_rows, n_q, max_kv_len, topk, topk_idx, topk_score};
  if (topk_two_phase(n_q, max_kv_len)) {
    // few long rows: per-segment candidates after the scores
    t.n_seg = static_cast<int32_t>(ceil_div(max_kv_len, kTopkSegLen));
    t.seg_len = kTopkSegLen;
    uint8_t* base = static_cast<uint8_t*>(ws) + sizeof(float) * static_cast<size_t>(n_q) * stride;
    t.cand_score = reinterpret_cast<float*>(base);
    t.cand_pos = reinterpret_cast<int32_t*>(base + sizeof(float) * static_cast<size_t>(n_q) *
                                                     t.n_seg * kTopkMax);
  }
  return launch_topk(t, stream);
}

static ds_status check_mla(const char* fn, const MlaArgs& a) {
  const std::string f(fn);
  DS_REQUIRE(a.n_q >= 0 && a.kv_rows >= 0, DS_ERR_INVALID_ARG, f + ": negative size");
  DS_REQUIRE(a.topk >= 1 && a.topk <= 2048, DS_ERR_INVALID_ARG, f + ": topk must be in [1, 2048]");
  DS_REQUIRE(a.n_heads >= 1 && a.d_latent >= 1 && a.d_rope >= 0, DS_ERR_INVALID_ARG,
             f + ": bad head/latent dims");
  DS_REQUIRE(a.sm_scale > 0.f && a.sm_scale <= 3.4e38f, DS_ERR_INVALID_ARG,
             f + ": sm_scale must be positive and finite");
  if (a.n_q > 0)
    DS_REQUIRE(a.q && a.topk_idx && a.out && (a.kv_rows == 0 || a.kv), DS_ERR_INVALID_ARG,
               f + ": NULL q/kv/topk_idx/out");
  DS_REQUIRE(a.out_dtype == DS_F32 || a.out_dtype == DS_BF16, DS_ERR_UNSUPPORTED,
             f + ": out must be f32 or bf16");
  if (a.q_dtype == DS_F32) {
    DS_REQUIRE(a.kv_dtype == DS_F32 && a.out_dtype == DS_F32, DS_ERR_UNSUPPORTED,
               f + ": f32 queries need f32 kv and f32 out");
    DS_REQUIRE(a.n_heads <= 128 && a.d_latent + a.d_rope <= 640, DS_ERR_UNSUPPORTED,
               f + ": f32 path supports n_heads <= 128, d_latent + d_rope <= 640");
  } else if (a.q_dtype == DS_BF16) {
    DS_REQUIRE(a.kv_dtype == DS_BF16 || a.kv_dtype == DS_FP8_E4M3FN ||
                   a.kv_dtype == DS_FP8_E4M3FN_ROWSCALE,
               DS_ERR_UNSUPPORTED, f + ": bf16 queries need bf16 or fp8 kv");
    // the kernels run 32, 64 or 128 heads per query row (a 96-head row
    // would have them read and write a neighbouring row's heads)
    DS_REQUIRE((a.n_heads == 32 || a.n_heads == 64 || a.n_heads == 128) && a.d_latent == 512 &&
                   a.d_rope == 64,
               DS_ERR_UNSUPPORTED,
               f + ": bf16 path supports n_heads 32, 64 or 128, d_latent 512, d_rope 64");
  } else {
    return fail(DS_ERR_UNSUPPORTED, f + ": q must be f32 or bf16");
  }
  if (a.kv_dtype == DS_FP8_E4M3FN || a.kv_dtype == DS_FP8_E4M3FN_ROWSCALE)
    DS_REQUIRE(a.kv_scale != nullptr, DS_ERR_INVALID_ARG, f + ": fp8 kv needs kv_scale");
  return DS_OK;
}

size_t sparse_mla_prefill_workspace_size(int64_t kv_rows, ds_dtype kv_dtype) {
  if ((kv_dtype != DS_FP8_E4M3FN && kv_dtype != DS_FP8_E4M3FN_ROWSCALE) || kv_rows <= 0) return 0;
  return static_cast<size_t>(kv_rows) * kMlaWidenedRowBytes;
}

ds_status sparse_mla_prefill(const void* q, ds_dtype q_dtype, const void* kv,
                             ds_dtype kv_dtype, const float* kv_scale, int64_t kv_rows,
                             const int32_t* topk_idx, int32_t n_q, int32_t n_heads,
                             int32_t d_latent, int32_t d_rope, int32_t topk,
                             float sm_scale, void* out, ds_dtype out_dtype, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  MlaArgs a{q, q_dtype, kv, kv_dtype, kv_scale, kv_rows, topk_idx, n_q, n_heads, d_latent,
            d_rope, topk, sm_scale, out, out_dtype, lse, 1, nullptr};
  ds_status st = check_mla("sparse_mla_prefill", a);
  if (st != DS_OK) return st;
  normalize_fp8(a);
  const size_t need = sparse_mla_prefill_workspace_size(kv_rows, kv_dtype);
  if (need > 0) {
    DS_REQUIRE(ws != nullptr && ws_bytes >= need, DS_ERR_WORKSPACE,
               "sparse_mla_prefill: fp8 kv needs sparse_mla_prefill_workspace_size() bytes of workspace");
    DS_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, DS_ERR_INVALID_ARG,
               "sparse_mla_prefill: workspace must be 256-byte aligned");
    st = launch_widen_fp8_rows(kv, kv_scale, a.scale_shift, kv_rows, ws, stream);
    if (st != DS_OK) return st;
    a.kv = ws;
    a.kv_dtype = DS_BF16;
    a.kv_scale = nullptr;
  }
  return launch_sparse_mla(a, stream);
}

size_t sparse_mla_workspace_size(int32_t n_q, int32_t n_heads, int32_t d_latent,
                                 int32_t topk) {
  if (n_q <= 0 || n_heads <= 0 || d_latent <= 0 || topk <= 0) return 256;
  return mla_partials_bytes(n_q, n_heads, d_latent, mla_decode_splits(n_q, topk));
}

ds_status sparse_mla_decode(const void* q, ds_dtype q_dtype, const void* kv,
                            ds_dtype kv_dtype, const float* kv_scale, int64_t kv_rows,
                            const int32_t* topk_idx, int32_t n_q, int32_t n_heads,
                            int32_t d_latent, int32_t d_rope, int32_t topk, float sm_scale,
                            void* out, ds_dtype out_dtype, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  MlaArgs a{q, q_dtype, kv, kv_dtype, kv_scale, kv_rows, topk_idx, n_q, n_heads, d_latent,
            d_rope, topk, sm_scale, out, out_dtype, lse, 1, ws};
  ds_status st = check_mla("sparse_mla_decode", a);
  if (st != DS_OK) return st;
  normalize_fp8(a);
  DS_REQUIRE(ws != nullptr && ws_bytes >= sparse_mla_workspace_size(n_q, n_heads, d_latent, topk),
             DS_ERR_WORKSPACE, "sparse_mla_decode: workspace smaller than sparse_mla_workspace_size()");
  if (q_dtype != DS_F32) a.n_splits = mla_decode_splits(n_q, topk);
  return launch_sparse_mla(a, stream);
}

size_t gemm_bf16_nt_workspace_size(int32_t M, int32_t N, int32_t K, int32_t batch) {
  if (M <= 0 || N <= 0 || K <= 0 || batch <= 0) return 0;
  const int32_t splits = gemm_splits(M, N, K, batch);
  return splits > 1 ? sizeof(float) * static_cast<size_t>(splits) * batch * M * N : 0;
}

ds_status gemm_bf16_nt(const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                       int64_t stride_b, void* C, ds_dtype c_dtype, int64_t ldc, int64_t stride_c,
                       int32_t M, int32_t N, int32_t K, int32_t batch, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  const char* f = "gemm_bf16_nt";
  DS_REQUIRE(M >= 0 && N >= 0 && K >= 0 && batch >= 0, DS_ERR_INVALID_ARG,
             std::string(f) + ": negative size");
  DS_REQUIRE(c_dtype == DS_BF16 || c_dtype == DS_F32, DS_ERR_UNSUPPORTED,
             std::string(f) + ": C must be bf16 or f32");
  DS_REQUIRE(K % 64 == 0 && N % 128 == 0, DS_ERR_UNSUPPORTED,
             std::string(f) + ": K must be a multiple of 64 and N of 128");
  if (static_cast<int64_t>(M) * N * batch == 0) return DS_OK;
  DS_REQUIRE(A != nullptr && B != nullptr && C != nullptr, DS_ERR_INVALID_ARG,
             std::string(f) + ": NULL operand");
  DS_REQUIRE(lda >= K && ldb >= K && ldc >= N && stride_a >= 0 && stride_b >= 0 && stride_c >= 0,
             DS_ERR_INVALID_ARG, std::string(f) + ": leading dimensions below the row length");
  DS_REQUIRE(((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0 &&
                 (lda | ldb | stride_a | stride_b) % 8 == 0,
             DS_ERR_INVALID_ARG,
             std::string(f) + ": A and B need 16-byte aligned rows (pointers, strides % 8)");
  GemmArgs g{A, B, C, ws, lda, ldb, ldc, stride_a, stride_b, stride_c, M, N, K, batch, 1, c_dtype};
  g.splits = gemm_splits(M, N, K, batch);
  if (g.splits > 1)
    DS_REQUIRE(ws != nullptr && ws_bytes >= gemm_bf16_nt_workspace_size(M, N, K, batch),
               DS_ERR_WORKSPACE, std::string(f) + ": workspace smaller than gemm_bf16_nt_workspace_size()");
  return launch_gemm(g, stream);
}

size_t sparse_mla_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

ds_status sparse_mla_decode_noalloc(const void* q, ds_dtype q_dtype, const void* kv,
                                    ds_dtype kv_dtype, const float* kv_scale, int64_t kv_rows,
                                    const int32_t* topk_idx, int32_t n_q, int32_t n_heads,
                                    int32_t d_latent, int32_t d_rope, int32_t topk,
                                    float sm_scale, void* out, ds_dtype out_dtype, float* lse,
                                    hipStream_t stream) {
  MlaArgs a{q, q_dtype, kv, kv_dtype, kv_scale, kv_rows, topk_idx, n_q, n_heads, d_latent,
            d_rope, topk, sm_scale, out, out_dtype, lse, 1, nullptr};
  ds_status st = check_mla("sparse_mla_decode_noalloc", a);
  if (st != DS_OK) return st;
  normalize_fp8(a);
  if (q_dtype == DS_F32 || n_q == 0) return launch_sparse_mla(a, stream);   // no partials
  // the default split count when its partials fit the scratch, else the
  // largest count that does (one split writes the output directly)
  int32_t splits = mla_decode_splits(n_q, topk);
  while (splits > 1 && mla_partials_bytes(n_q, n_heads, d_latent, splits) > kNoAllocScratchBytes)
    --splits;
  if (splits > 1) {
    DS_REQUIRE(mla_partials_bytes(n_q, n_heads, d_latent, splits) <= kNoAllocScratchBytes,
               DS_ERR_WORKSPACE, "sparse_mla_decode_noalloc: partials exceed the scratch");
    st = scratch_ptr(&a.ws);
    if (st != DS_OK) return st;
  }
  a.n_splits = splits;
  return launch_sparse_mla(a, stream);
}

}  // extern "C"
