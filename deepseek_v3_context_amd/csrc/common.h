// Internal helpers shared by the ds32cp HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "ds32cp.h"

namespace ds32cp {

// ----------------------------------------------------------------- errors
// Per-thread last error text (read through ds_last_error()).
void set_error(const std::string& msg);
ds_status fail(ds_status code, const std::string& msg);
// Checks the launch that just happened on the calling thread.
ds_status check_launch(const char* what);

// Compute units of the current device (cached per device).
int32_t device_cu_count();

// ----------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxDevices = 64;   // per-device host caches
constexpr int kFp8BlockRows = 128;
constexpr int kCacheFp8MaxElems = 1024;   // kv_cache_write_fp8: elements per row

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (NaN stays NaN): gfx950's
// conversion instruction (v_cvt_pk_bf16_f32, two values per instruction
// when the compiler pairs them) instead of the integer rounding sequence.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two OCP e4m3fn codes (bytes 0,1 of `word`, or bytes 2,3 when kHi) ->
// two floats.  gfx950's conversion instructions use the OCP formats.
template <bool kHi>
__device__ __forceinline__ float2 fp8x2_to_f32(uint32_t word) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f r = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), kHi);
  return make_float2(r.x, r.y);
}

// Four e4m3fn codes -> four bfloat16 bit patterns, exactly: every e4m3fn
// value is representable in bfloat16, and gfx950's packed conversion with a
// unit scale gives those values (checked on the device against the two-step
// conversion through fp32 for every code in every byte position).
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t word) {
  uint2 out;
  out.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
  out.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
  return out;
}

// Order-preserving map float -> uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------ XCD mapping
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap a linear workgroup id so that XCD x receives a contiguous run
// of logical ids: ids that share operands then share that XCD's L2.
// `grid` must be a multiple of 8.
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t bid, uint32_t grid) {
  const uint32_t per_xcd = grid >> 3;
  return (bid & 7u) * per_xcd + (bid >> 3);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// --------------------------------------------------------- launch helpers
// (declared here, defined in the kernel sources; all return ds_status)
ds_status launch_split_metadata(const int32_t* cu, int32_t B, int32_t T, int32_t cp,
                                int32_t r, int32_t n, int32_t* local_cu,
                                int32_t* batch_idx, int32_t* global_idx,
                                int32_t* kv_start, int32_t* kv_len,
                                hipStream_t s);
ds_status launch_in_seq_split(const int32_t* cu, int32_t B, int32_t T, int32_t cp, int32_t r,
                              int32_t n, int32_t* local_cu, int32_t* batch_idx,
                              int32_t* global_idx, int32_t* kv_start, int32_t* kv_len,
                              const void* rows_src, void* rows_dst, int64_t row_bytes,
                              hipStream_t s);
ds_status launch_decode_metadata(const int32_t* lengths, int32_t n, int32_t* q_req,
                                 int32_t* kv_start, int32_t* kv_len, hipStream_t s);
ds_status launch_row_gather_rr(const void* src, void* dst, int32_t n, int32_t cp,
                               int32_t r, int64_t row_bytes, hipStream_t s);
ds_status launch_rerange(const void* src, void* dst, int32_t T, int32_t cp,
                         int32_t slot_rows, int64_t row_bytes, hipStream_t s);
ds_status launch_kv_cache_write_fp8(const void* rows, int32_t n_local, int32_t row_elems,
                                    const int32_t* batch_idx, const int32_t* local_cu,
                                    int32_t n_req, const int32_t* page_table, int32_t max_pages,
                                    int32_t page_size, uint8_t* pool_codes, float* pool_scale,
                                    int64_t pool_rows, hipStream_t s);
ds_status launch_kv_cache_write(const void* rows, int32_t n_local, int64_t row_bytes,
                                const int32_t* batch_idx, const int32_t* local_cu,
                                int32_t n_req, const int32_t* page_table,
                                int32_t max_pages, int32_t page_size, void* pool,
                                int64_t pool_rows, hipStream_t s);

struct IndexerArgs {
  const void* q_idx;
  ds_dtype q_dtype;
  const float* w;
  const void* k_idx;
  ds_dtype k_dtype;
  const float* k_scale;
  int64_t k_rows;
  const int32_t* kv_start;
  const int32_t* kv_len;
  const int32_t* q_req;
  const int32_t* page_table;
  int32_t n_req, page_size, max_pages;
  int32_t n_q, h_idx, d_idx, max_kv_len;
  float* scores;
  int64_t score_stride;
  int32_t k_scale_shift = 7;   // fp8 keys: scale of row r is k_scale[r >> k_scale_shift]
};
ds_status launch_indexer_scores(const IndexerArgs& a, hipStream_t s);

struct TopkArgs {
  const float* scores;
  int64_t score_stride;
  const int32_t* kv_start;
  const int32_t* kv_len;
  const int32_t* q_req;
  const int32_t* page_table;
  int32_t n_req, page_size, max_pages;
  int64_t k_rows;
  int32_t n_q, max_kv_len, topk;
  int32_t* topk_idx;
  float* topk_score;
  // two-phase selection of long rows (see topk.hip): per-segment
  // candidates, n_seg segments of seg_len positions per row, topk each
  float* cand_score = nullptr;
  int32_t* cand_pos = nullptr;
  int32_t n_seg = 0, seg_len = 0;
};
ds_status launch_topk(const TopkArgs& a, hipStream_t s);
// fp8 latent rows (576 codes, scale per 128 rows) -> bf16 rows (code * scale)
constexpr int kMlaWidenedRowBytes = 576 * 2;
ds_status launch_widen_fp8_rows(const void* codes, const float* scale, int32_t scale_shift,
                                int64_t rows, void* out, hipStream_t s);
// Few rows longer than the single-workgroup bitmap selection takes (65536
// keys) are selected in two phases, over segments of kTopkSegLen keys and
// then over the segments' candidates (topk_two_phase_bytes() of workspace).
constexpr int32_t kTopkSegLen = 8192;
constexpr int32_t kTopkMax = 2048;
constexpr int32_t kTopkOnePassMaxLen = 65536;
inline bool topk_two_phase(int32_t n_q, int32_t max_kv_len) {
  return max_kv_len > kTopkOnePassMaxLen && n_q <= 256;
}
inline size_t topk_two_phase_bytes(int32_t n_q, int32_t max_kv_len) {
  const int64_t n_seg = (static_cast<int64_t>(max_kv_len) + kTopkSegLen - 1) / kTopkSegLen;
  return static_cast<size_t>(n_q) * n_seg * kTopkMax * (sizeof(float) + sizeof(int32_t));
}

struct MlaArgs {
  const void* q;
  ds_dtype q_dtype;
  const void* kv;
  ds_dtype kv_dtype;
  const float* kv_scale;
  int64_t kv_rows;
  const int32_t* topk_idx;
  int32_t n_q, n_heads, d_latent, d_rope, topk;
  float sm_scale;
  void* out;
  ds_dtype out_dtype;
  float* lse;
  int32_t n_splits;   // > 1: split each query's rows (decode variant)
  void* ws;           // partials for n_splits > 1
  int32_t scale_shift = 7;   // fp8 kv: scale of row r is kv_scale[r >> scale_shift]
};
ds_status launch_sparse_mla(const MlaArgs& a, hipStream_t s);

// Batched C = A . B^T (the projections); strides in elements.
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  void* ws;                       // split-K partials (fp32), splits > 1
  int64_t lda, ldb, ldc;
  int64_t strideA, strideB, strideC;
  int32_t M, N, K, batch, splits;
  ds_dtype c_dtype;
};
int32_t gemm_splits(int32_t M, int32_t N, int32_t K, int32_t batch);
ds_status launch_gemm(GemmArgs g, hipStream_t s);
size_t mla_partials_bytes(int32_t n_q, int32_t n_heads, int32_t d_latent,
                          int32_t n_splits);
int32_t mla_decode_splits(int32_t n_q, int32_t topk);

}  // namespace ds32cp
