// Step 1 (round-robin split + metadata) and step 2 (KV rerange).
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

// dst row j <- src row src_row(j), vectors of type V.
struct GatherRR {  // split: dst j <- src r + j*cp
  int32_t cp, r;
  __device__ int64_t operator()(int64_t j) const { return r + j * cp; }
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
    dst[e] = src[map(row) * vecs_per_row + col];
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

ds_status launch_rerange(const void* src, void* dst, int32_t T, int32_t cp,
                         int32_t slot_rows, int64_t row_bytes, hipStream_t s) {
  return launch_permute(src, dst, T, row_bytes, Rerange{cp, slot_rows}, s,
                        "kv_rerange");
}

}  // namespace ds32cp
