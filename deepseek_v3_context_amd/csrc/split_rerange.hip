// Step 1 (round-robin split + metadata; the in-sequence split it replaces,
// for contrast) and step 2 (KV rerange).
//
// Sources: "[DeepSeek v3.2] 上下文并行详解", section 1 and section 2B
// (token g goes to rank g mod cp_size; the rank's sequence lengths, batch
// indices and cumulative offsets are recomputed), section 4 part 3 steps 1
// and B (rank-concatenated rows are put back into logical order), and the
// causal example of step C (position p sees positions 0..p).
//
// Both are HBM-bound permutations.  Rows move as 16-, 8-, 4- or 1-byte
// vectors, chosen on the host from the row size and pointer alignment;
// consecutive threads move consecutive vectors of the destination so that
// writes are fully coalesced and each source row is read contiguously.
#include "common.h"

namespace ds32cp {

// One thread per output element of each array (n queries, B+1 offsets).
__global__ void __launch_bounds__(256)
split_metadata_kernel(const int32_t* __restrict__ cu, int32_t B, int32_t T,
                      int32_t cp, int32_t r, int32_t n,
                      int32_t* __restrict__ local_cu,
                      int32_t* __restrict__ batch_idx,
                      int32_t* __restrict__ global_idx,
                      int32_t* __restrict__ kv_start,
                      int32_t* __restrict__ kv_len) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (local_cu && i <= B) {
    // count of g < cu[i] with g = r (mod cp)
    const int32_t x = cu[i];
    local_cu[i] = x > r ? (x - r + cp - 1) / cp : 0;
  }
  if (i < n) {
    const int32_t g = r + i * cp;
    // request b: the last b in [0, B) with cu[b] <= g (empty requests are
    // skipped because a later equal offset wins)
    int32_t lo = 0, hi = B - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int32_t start = cu[lo];
    if (batch_idx) batch_idx[i] = lo;
    if (global_idx) global_idx[i] = g;
    if (kv_start) kv_start[i] = start;
    if (kv_len) kv_len[i] = g - start + 1;
  }
}

// ------------------------------------------------------------------
// In-sequence split (the contrast mode of the same page, section 4 part 1):
// request b of L_b tokens is cut into chunks of c_b = ceil(L_b / cp) tokens
// and rank r takes chunk r, positions [r c_b, min(L_b, (r+1) c_b)).
__device__ __forceinline__ int32_t in_seq_chunk(int32_t len, int32_t cp) {
  return static_cast<int32_t>((static_cast<int64_t>(len) + cp - 1) / cp);
}
__device__ __forceinline__ int32_t in_seq_count(int32_t len, int32_t cp, int32_t r) {
  const int64_t c = in_seq_chunk(len, cp);
  const int64_t left = static_cast<int64_t>(len) - r * c;
  return static_cast<int32_t>(left <= 0 ? 0 : (left < c ? left : c));
}

// local_cu[b] = the rank's tokens in requests before b: one workgroup scans
// the per-request counts 1024 at a time (wave scans with row shuffles, then
// across the 16 waves), carrying the running total between rounds.
__global__ void __launch_bounds__(1024)
in_seq_local_cu_kernel(const int32_t* __restrict__ cu, int32_t B, int32_t cp, int32_t r,
                       int32_t* __restrict__ local_cu) {
  __shared__ int32_t wave_sum[1024 / kWave];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    carry = 0;
    local_cu[0] = 0;
  }
  __syncthreads();
  for (int32_t base = 0; base < B; base += 1024) {
    const int32_t b = base + tid;
    int32_t v = b < B ? in_seq_count(cu[b + 1] - cu[b], cp, r) : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t u = __shfl_up(v, off);
      if (lane >= off) v += u;
    }
    if (lane == kWave - 1) wave_sum[wave] = v;
    __syncthreads();
    int32_t before = carry;
    for (int w = 0; w < wave; ++w) before += wave_sum[w];
    if (b < B) local_cu[b + 1] = before + v;
    __syncthreads();
    if (tid == 1023) carry = before + v;
    __syncthreads();
  }
}

// One thread per local token j: its request b (the last b with
// local_cu[b] <= j, so empty requests are skipped), position
// p = r c_b + (j - local_cu[b]), global index cu[b] + p.  Entries past the
// rank's token count (when the caller's n exceeds it) get batch and global
// index -1 and an empty causal range.
__global__ void __launch_bounds__(256)
in_seq_token_kernel(const int32_t* __restrict__ cu, int32_t B, int32_t cp, int32_t r, int32_t n,
                    const int32_t* __restrict__ local_cu, int32_t* __restrict__ batch_idx,
                    int32_t* __restrict__ global_idx, int32_t* __restrict__ kv_start,
                    int32_t* __restrict__ kv_len) {
  const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  if (j >= local_cu[B]) {
    if (batch_idx) batch_idx[j] = -1;
    if (global_idx) global_idx[j] = -1;
    if (kv_start) kv_start[j] = 0;
    if (kv_len) kv_len[j] = 0;
    return;
  }
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (local_cu[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int32_t p = r * in_seq_chunk(cu[lo + 1] - cu[lo], cp) + (j - local_cu[lo]);
  if (batch_idx) batch_idx[j] = lo;
  if (global_idx) global_idx[j] = cu[lo] + p;
  if (kv_start) kv_start[j] = cu[lo];
  if (kv_len) kv_len[j] = p + 1;
}

// dst row j <- src row src_row(j), vectors of type V (rows mapped to a
// negative index are skipped).
struct GatherRR {  // split: dst j <- src r + j*cp
  int32_t cp, r;
  __device__ int64_t operator()(int64_t j) const { return r + j * cp; }
};
struct GatherIdx {   // in-sequence split: dst j <- src idx[j] (skipped outside [0, limit))
  const int32_t* idx;
  int32_t limit;
  __device__ int64_t operator()(int64_t j) const {
    const int32_t g = idx[j];
    return (g >= 0 && g < limit) ? g : -1;
  }
};
struct Rerange {   // rerange: dst g <- src (g mod cp)*slot + g div cp
  int32_t cp, slot;
  __device__ int64_t operator()(int64_t g) const {
    return static_cast<int64_t>(g % cp) * slot + g / cp;
  }
};

template <typename V, typename Map>
__global__ void __launch_bounds__(256)
row_permute_kernel(const V* __restrict__ src, V* __restrict__ dst,
                   int64_t n_rows, int64_t vecs_per_row, Map map) {
  const int64_t total = n_rows * vecs_per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       e < total; e += stride) {
    const int64_t row = e / vecs_per_row;
    const int64_t col = e - row * vecs_per_row;
    const int64_t from = map(row);
    if (from >= 0) dst[e] = src[from * vecs_per_row + col];
  }
}

template <typename Map>
static ds_status launch_permute(const void* src, void* dst, int64_t n_rows,
                                int64_t row_bytes, Map map, hipStream_t s,
                                const char* what) {
  if (n_rows == 0) return DS_OK;
  const uintptr_t al = reinterpret_cast<uintptr_t>(src) |
                       reinterpret_cast<uintptr_t>(dst) |
                       static_cast<uintptr_t>(row_bytes);
  int vec = 1;
  if ((al & 15) == 0) vec = 16;
  else if ((al & 7) == 0) vec = 8;
  else if ((al & 3) == 0) vec = 4;
  const int64_t vpr = row_bytes / vec;
  const int64_t total = n_rows * vpr;
  const int threads = 256;
  const int64_t want = ceil_div(total, threads);
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  switch (vec) {
    case 16:
      row_permute_kernel<uint4, Map><<<blocks, threads, 0, s>>>(
          static_cast<const uint4*>(src), static_cast<uint4*>(dst), n_rows, vpr, map);
      break;
    case 8:
      row_permute_kernel<uint2, Map><<<blocks, threads, 0, s>>>(
          static_cast<const uint2*>(src), static_cast<uint2*>(dst), n_rows, vpr, map);
      break;
    case 4:
      row_permute_kernel<uint32_t, Map><<<blocks, threads, 0, s>>>(
          static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), n_rows, vpr, map);
      break;
    default:
      row_permute_kernel<uint8_t, Map><<<blocks, threads, 0, s>>>(
          static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), n_rows, vpr, map);
  }
  return check_launch(what);
}

// Own-KV retention: local row j, of request b = batch_idx[j] and cache
// position p = j - local_cu[b], goes to pool row page_table[b][p / ps] * ps
// + p % ps; a row that maps to no pool row is skipped.  One vector of V per
// thread and step; every thread recomputes its row's destination (a few
// cached loads) so that rows of any length need no cooperation.
template <typename V>
__global__ void __launch_bounds__(256)
kv_cache_write_kernel(const V* __restrict__ src, V* __restrict__ pool, int64_t n_rows,
                      int64_t vecs_per_row, const int32_t* __restrict__ batch_idx,
                      const int32_t* __restrict__ local_cu, int32_t n_req,
                      const int32_t* __restrict__ page_table, int32_t max_pages,
                      int32_t page_size, int64_t pool_rows) {
  const int64_t total = n_rows * vecs_per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       e < total; e += stride) {
    const int64_t j = e / vecs_per_row;
    const int64_t col = e - j * vecs_per_row;
    const int32_t b = batch_idx[j];
    if (b < 0 || b >= n_req) continue;
    const int64_t p = j - local_cu[b];
    if (p < 0) continue;
    const int64_t pg = p / page_size;
    if (pg >= max_pages) continue;
    const int32_t page = page_table[static_cast<int64_t>(b) * max_pages + pg];
    if (page < 0) continue;
    const int64_t phys = static_cast<int64_t>(page) * page_size + (p - pg * page_size);
    if (phys >= pool_rows) continue;
    pool[phys * vecs_per_row + col] = src[e];
  }
}

// Own-KV retention with fp8 encoding: one wave per local row (the same
// destination rule as kv_cache_write_kernel), four consecutive bf16 values
// per lane and step (row_elems <= 1024: at most four steps, held in
// registers).  scale = row amax / 448 (a correctly rounded fp32 division),
// code = e4m3fn of clamp(x / scale, +-448) by gfx950's conversion
// instruction (round to nearest even); an all-zero row stores scale 0 and
// zero codes.
__global__ void __launch_bounds__(256)
kv_cache_write_fp8_kernel(const uint16_t* __restrict__ rows, int32_t n_local, int32_t D,
                          const int32_t* __restrict__ batch_idx,
                          const int32_t* __restrict__ local_cu, int32_t n_req,
                          const int32_t* __restrict__ page_table, int32_t max_pages,
                          int32_t page_size, uint8_t* __restrict__ codes,
                          float* __restrict__ scales, int64_t pool_rows) {
  constexpr float kE4m3Max = 448.f;
  const int lane = threadIdx.x & 63;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  // every exit below is uniform over the wave (one row per wave)
  if (j >= n_local) return;
  const int32_t b = batch_idx[j];
  if (b < 0 || b >= n_req) return;
  const int64_t p = j - local_cu[b];
  if (p < 0) return;
  const int64_t pg = p / page_size;
  if (pg >= max_pages) return;
  const int32_t page = page_table[static_cast<int64_t>(b) * max_pages + pg];
  if (page < 0) return;
  const int64_t phys = static_cast<int64_t>(page) * page_size + (p - pg * page_size);
  if (phys >= pool_rows) return;
  const int G = D >> 2;   // groups of four values
  float x[4][4];
  float amax = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int g = lane + kWave * s;
    uint2 v = make_uint2(0u, 0u);
    if (g < G) v = *reinterpret_cast<const uint2*>(rows + j * D + 4 * g);
    x[s][0] = bf16_bits_to_f32(static_cast<uint16_t>(v.x & 0xffffu));
    x[s][1] = bf16_bits_to_f32(static_cast<uint16_t>(v.x >> 16));
    x[s][2] = bf16_bits_to_f32(static_cast<uint16_t>(v.y & 0xffffu));
    x[s][3] = bf16_bits_to_f32(static_cast<uint16_t>(v.y >> 16));
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(x[s][e]));
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax / kE4m3Max;
  if (lane == 0) scales[phys] = scale;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int g = lane + kWave * s;
    if (g >= G) continue;
    uint32_t word = 0u;
    if (scale > 0.f) {
      float q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(x[s][e] / scale, -kE4m3Max), kE4m3Max);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
      word = static_cast<uint32_t>(w);
    }
    *reinterpret_cast<uint32_t*>(codes + phys * D + 4 * g) = word;
  }
}

ds_status launch_kv_cache_write_fp8(const void* rows, int32_t n_local, int32_t row_elems,
                                    const int32_t* batch_idx, const int32_t* local_cu,
                                    int32_t n_req, const int32_t* page_table, int32_t max_pages,
                                    int32_t page_size, uint8_t* pool_codes, float* pool_scale,
                                    int64_t pool_rows, hipStream_t s) {
  if (n_local == 0) return DS_OK;
  kv_cache_write_fp8_kernel<<<static_cast<unsigned>(ceil_div(n_local, 4)), 256, 0, s>>>(
      static_cast<const uint16_t*>(rows), n_local, row_elems, batch_idx, local_cu, n_req,
      page_table, max_pages, page_size, pool_codes, pool_scale, pool_rows);
  return check_launch("kv_cache_write_fp8");
}

ds_status launch_kv_cache_write(const void* rows, int32_t n_local, int64_t row_bytes,
                                const int32_t* batch_idx, const int32_t* local_cu,
                                int32_t n_req, const int32_t* page_table,
                                int32_t max_pages, int32_t page_size, void* pool,
                                int64_t pool_rows, hipStream_t s) {
  if (n_local == 0) return DS_OK;
  const uintptr_t al = reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(pool) |
                       static_cast<uintptr_t>(row_bytes);
  int vec = 1;
  if ((al & 15) == 0) vec = 16;
  else if ((al & 7) == 0) vec = 8;
  else if ((al & 3) == 0) vec = 4;
  const int64_t vpr = row_bytes / vec;
  const int64_t total = static_cast<int64_t>(n_local) * vpr;
  const int threads = 256;
  const int64_t want = ceil_div(total, threads);
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
#define DS_KVW(V)                                                                        \
  kv_cache_write_kernel<V><<<blocks, threads, 0, s>>>(                                   \
      static_cast<const V*>(rows), static_cast<V*>(pool), n_local, vpr, batch_idx,       \
      local_cu, n_req, page_table, max_pages, page_size, pool_rows)
  switch (vec) {
    case 16: DS_KVW(uint4); break;
    case 8: DS_KVW(uint2); break;
    case 4: DS_KVW(uint32_t); break;
    default: DS_KVW(uint8_t);
  }
#undef DS_KVW
  return check_launch("kv_cache_write");
}

ds_status launch_split_metadata(const int32_t* cu, int32_t B, int32_t T, int32_t cp,
                                int32_t r, int32_t n, int32_t* local_cu,
                                int32_t* batch_idx, int32_t* global_idx,
                                int32_t* kv_start, int32_t* kv_len,
                                hipStream_t s) {
  const int32_t items = (n > B + 1) ? n : B + 1;
  const int threads = 256;
  const unsigned blocks = static_cast<unsigned>(ceil_div(items, threads));
  split_metadata_kernel<<<blocks, threads, 0, s>>>(cu, B, T, cp, r, n, local_cu,
                                                   batch_idx, global_idx,
                                                   kv_start, kv_len);
  return check_launch("cp_split_metadata");
}

ds_status launch_row_gather_rr(const void* src, void* dst, int32_t n, int32_t cp,
                               int32_t r, int64_t row_bytes, hipStream_t s) {
  return launch_permute(src, dst, n, row_bytes, GatherRR{cp, r}, s,
                        "cp_split_metadata row gather");
}

ds_status launch_in_seq_split(const int32_t* cu, int32_t B, int32_t T, int32_t cp, int32_t r,
                              int32_t n, int32_t* local_cu, int32_t* batch_idx,
                              int32_t* global_idx, int32_t* kv_start, int32_t* kv_len,
                              const void* rows_src, void* rows_dst, int64_t row_bytes,
                              hipStream_t s) {
  in_seq_local_cu_kernel<<<1, 1024, 0, s>>>(cu, B, cp, r, local_cu);
  ds_status st = check_launch("cp_split_metadata_in_seq (offsets)");
  if (st != DS_OK || n == 0) return st;
  in_seq_token_kernel<<<static_cast<unsigned>(ceil_div(n, 256)), 256, 0, s>>>(
      cu, B, cp, r, n, local_cu, batch_idx, global_idx, kv_start, kv_len);
  st = check_launch("cp_split_metadata_in_seq");
  if (st != DS_OK || rows_src == nullptr) return st;
  return launch_permute(rows_src, rows_dst, n, row_bytes, GatherIdx{global_idx, T}, s,
                        "cp_split_metadata_in_seq row gather");
}

// Decode step metadata: request i has one query at position L_i - 1 whose
// causal keys are positions 0 .. L_i - 1 of the request (its own KV is
// already cached); negative lengths give an empty range.
__global__ void __launch_bounds__(256)
decode_metadata_kernel(const int32_t* __restrict__ lengths, int32_t n, int32_t* __restrict__ q_req,
                       int32_t* __restrict__ kv_start, int32_t* __restrict__ kv_len) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t L = lengths[i];
  if (q_req) q_req[i] = i;
  if (kv_start) kv_start[i] = 0;
  if (kv_len) kv_len[i] = L > 0 ? L : 0;
}

ds_status launch_decode_metadata(const int32_t* lengths, int32_t n, int32_t* q_req,
                                 int32_t* kv_start, int32_t* kv_len, hipStream_t s) {
  if (n == 0) return DS_OK;
  decode_metadata_kernel<<<static_cast<unsigned>(ceil_div(n, 256)), 256, 0, s>>>(
      lengths, n, q_req, kv_start, kv_len);
  return check_launch("decode_metadata");
}

ds_status launch_rerange(const void* src, void* dst, int32_t T, int32_t cp,
                         int32_t slot_rows, int64_t row_bytes, hipStream_t s) {
  return launch_permute(src, dst, T, row_bytes, Rerange{cp, slot_rows}, s,
                        "kv_rerange");
}

}  // namespace ds32cp
