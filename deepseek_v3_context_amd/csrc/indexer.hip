// Step 3: indexer scores.
//
// Sources: "[RFC]: Parallel strategy for Deepseek v3.2 like models",
// comment thread (the indexer is a per-query pass over the query's history
// that selects its top-k KV entries; it is the bottleneck that splitting
// queries over ranks shortens); "[DeepSeek v3.2] 上下文并行详解", section
// 2C (the indexer's KV range is taken on the logically ordered KV).
// Score reading (no formula on the pages):
//   I[j, p] = sum_h w[j, h] * max(0, <q_idx[j, h, :], k_idx[row(j, p), :]>)
//
// bf16/fp8 path (h_idx = 64, d_idx = 128): a dense contraction per
// (query, key) pair of 64 x 128 MACs, done on MFMA v_mfma_f32_32x32x16_bf16
// with heads as the M dimension and keys as N, so that one lane's output
// column is one key and the head reduction (after ReLU and the per-head
// weight) is 32 in-register FMAs plus one cross-half swap.
//   * prefill: a workgroup owns 8 consecutive queries (2 per wave, their
//     A fragments held in registers for the whole chunk) and a chunk of
//     absolute key rows; 32-key tiles are staged once in LDS and shared by
//     the 4 waves (double-buffered through registers).  Queries of one
//     workgroup may belong to different requests: each masks its own
//     causal range on write.
//   * decode: keys are paged per request, so a workgroup owns one query
//     and 256 logical positions (64 per wave) and reads B fragments
//     straight from HBM (each key row is read exactly once).
// fp8 keys are widened to bf16 exactly; the per-block scale is positive
// and multiplies the whole score of its key (ReLU commutes with a
// positive factor), so it is applied once per key after the head sum.
#include "common.h"

namespace ds32cp {

// Physical row of logical position l of request `req`, or -1.
__device__ __forceinline__ int64_t index_key_row(const IndexerArgs& a, int32_t req,
                                                 int64_t l) {
  if (l < 0) return -1;
  if (a.page_table == nullptr) return l < a.k_rows ? l : -1;
  const int64_t ps = a.page_size;
  const int64_t pg = l / ps;
  if (req < 0 || req >= a.n_req || pg >= a.max_pages) return -1;
  const int32_t pid = a.page_table[static_cast<int64_t>(req) * a.max_pages + pg];
  const int64_t row = static_cast<int64_t>(pid) * ps + (l - pg * ps);
  return (pid >= 0 && row < a.k_rows) ? row : -1;
}

__device__ __forceinline__ int32_t clamp_len(const IndexerArgs& a, int32_t j) {
  int32_t L = a.kv_len[j];
  L = L < 0 ? 0 : L;
  return L > a.max_kv_len ? a.max_kv_len : L;
}

// ---------------------------------------------------------------- fp32
// One thread per (query, position); the query's vectors sit in LDS.
__global__ void __launch_bounds__(256)
indexer_f32_kernel(IndexerArgs a) {
  extern __shared__ float smem[];
  float* qs = smem;                         // [h_idx * d_idx]
  float* ws = smem + a.h_idx * a.d_idx;     // [h_idx]
  const int32_t j = blockIdx.y;
  const int32_t L = clamp_len(a, j);
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (static_cast<int64_t>(blockIdx.x) * blockDim.x >= L) return;
  const float* q = static_cast<const float*>(a.q_idx) +
                   static_cast<int64_t>(j) * a.h_idx * a.d_idx;
  for (int i = threadIdx.x; i < a.h_idx * a.d_idx; i += blockDim.x) qs[i] = q[i];
  for (int i = threadIdx.x; i < a.h_idx; i += blockDim.x)
    ws[i] = a.w[static_cast<int64_t>(j) * a.h_idx + i];
  __syncthreads();
  if (p >= L) return;
  const int32_t req = a.q_req ? a.q_req[j] : 0;
  const int64_t row = index_key_row(a, req, a.kv_start[j] + p);
  float score = -INFINITY;
  if (row >= 0) {
    score = 0.f;
    for (int h = 0; h < a.h_idx; ++h) {
      float dot = 0.f;
      if (a.k_dtype == DS_F32) {
        const float* k = static_cast<const float*>(a.k_idx) + row * a.d_idx;
        for (int d = 0; d < a.d_idx; ++d) dot = fmaf(qs[h * a.d_idx + d], k[d], dot);
      } else {  // bf16 keys with f32 queries
        const uint16_t* k = static_cast<const uint16_t*>(a.k_idx) + row * a.d_idx;
        for (int d = 0; d < a.d_idx; ++d)
          dot = fmaf(qs[h * a.d_idx + d], bf16_bits_to_f32(k[d]), dot);
      }
      score = fmaf(ws[h], fmaxf(dot, 0.f), score);
    }
  }
  a.scores[static_cast<int64_t>(j) * a.score_stride + p] = score;
}

// ------------------------------------------------------- MFMA constants
constexpr int kIxHeads = 64;
constexpr int kIxDim = 128;
constexpr int kIxKSteps = kIxDim / 16;        // K = 16 per MFMA
constexpr int kIxRowBlocks = kIxHeads / 32;   // M = 32 per MFMA
constexpr int kIxWaves = 4;
constexpr int kIxQPerWave = 2;
constexpr int kIxQBlock = kIxWaves * kIxQPerWave;   // 8 queries / workgroup
constexpr int kIxTileKeys = 32;
constexpr int kIxRowBytes = kIxDim * 2 + 16;       // padded LDS row (bank spread)

// A fragment of v_mfma_f32_32x32x16_bf16 for heads [32*rb, 32*rb+32) and
// dims [16*ks, 16*ks+16): lane l holds head 32*rb + l%32, dims
// 16*ks + 8*(l/32) + 0..7 (16 contiguous bytes).
__device__ __forceinline__ bf16x8 load_q_frag(const uint16_t* q_row0, int rb, int ks,
                                              int lane) {
  const uint16_t* p = q_row0 + (rb * 32 + (lane & 31)) * kIxDim + ks * 16 + (lane >> 5) * 8;
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// Weighted ReLU head-sum of one 64-head x 32-key accumulator pair.  Output
// element i of lane l sits at head 8*(i/4) + 4*(l/32) + i%4 (+32*rb), key
// l%32; after the cross-half swap every lane holds its key's full sum.
__device__ __forceinline__ float head_sum(const f32x16 (&acc)[kIxRowBlocks],
                                          const float* w_heads, int lane) {
  float v = 0.f;
#pragma unroll
  for (int rb = 0; rb < kIxRowBlocks; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = rb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      v = fmaf(w_heads[h], fmaxf(acc[rb][i], 0.f), v);
    }
  }
  v += __shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------- prefill, MFMA path
template <bool kFp8>
__global__ void __launch_bounds__(256)
indexer_prefill_mfma_kernel(IndexerArgs a, int32_t n_qblocks, int32_t n_chunks,
                            int32_t chunk_keys, uint32_t grid) {
  __shared__ __align__(16) uint8_t ktile[2][kIxTileKeys * kIxRowBytes];
  __shared__ float wl[kIxQBlock][kIxHeads];
  __shared__ int64_t q_lo[kIxQBlock], q_hi[kIxQBlock];

  const uint32_t id = xcd_contiguous_id(blockIdx.x, grid);
  if (id >= static_cast<uint32_t>(n_qblocks) * n_chunks) return;
  const int32_t qb = id / n_chunks;
  const int32_t chunk = id - qb * n_chunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (tid < kIxQBlock) {
    const int32_t j = qb * kIxQBlock + tid;
    int64_t lo = 0, hi = 0;
    if (j < a.n_q) {
      lo = a.kv_start[j];
      hi = lo + clamp_len(a, j);
      if (lo < 0) lo = 0;
      if (hi > a.k_rows) hi = a.k_rows;
      if (hi < lo) hi = lo;
    }
    q_lo[tid] = lo;
    q_hi[tid] = hi;
  }
  for (int i = tid; i < kIxQBlock * kIxHeads; i += blockDim.x) {
    const int32_t j = qb * kIxQBlock + i / kIxHeads;
    wl[i / kIxHeads][i % kIxHeads] =
        j < a.n_q ? a.w[static_cast<int64_t>(j) * kIxHeads + i % kIxHeads] : 0.f;
  }
  __syncthreads();

  int64_t rlo = INT64_MAX, rhi = 0;
#pragma unroll
  for (int i = 0; i < kIxQBlock; ++i) {
    if (q_hi[i] > q_lo[i]) {
      rlo = q_lo[i] < rlo ? q_lo[i] : rlo;
      rhi = q_hi[i] > rhi ? q_hi[i] : rhi;
    }
  }
  const int64_t c_lo = static_cast<int64_t>(chunk) * chunk_keys;
  const int64_t c_hi = c_lo + chunk_keys;
  rlo = rlo > c_lo ? rlo : c_lo;
  rhi = rhi < c_hi ? rhi : c_hi;
  if (rlo >= rhi) return;
  const int64_t t_first = (rlo / kIxTileKeys) * kIxTileKeys;
  const int32_t n_tiles = static_cast<int32_t>(ceil_div(rhi - t_first, kIxTileKeys));

  // A fragments of this wave's two queries, resident for the whole chunk.
  bf16x8 qa[kIxQPerWave][kIxRowBlocks][kIxKSteps];
  int64_t my_lo[kIxQPerWave], my_hi[kIxQPerWave];
  int32_t my_j[kIxQPerWave];
#pragma unroll
  for (int s = 0; s < kIxQPerWave; ++s) {
    const int qi = wave * kIxQPerWave + s;
    my_j[s] = qb * kIxQBlock + qi;
    my_lo[s] = q_lo[qi];
    my_hi[s] = q_hi[qi];
    const bool live = my_hi[s] > my_lo[s];
    const uint16_t* q0 = static_cast<const uint16_t*>(a.q_idx) +
                         static_cast<int64_t>(live ? my_j[s] : 0) * kIxHeads * kIxDim;
#pragma unroll
    for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
      for (int ks = 0; ks < kIxKSteps; ++ks)
        qa[s][rb][ks] = live ? load_q_frag(q0, rb, ks, lane)
                             : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }

  // Cooperative tile load: bf16 keys 32 x 256 B (two 16-byte pieces per
  // thread); fp8 keys 32 x 128 B (one 16-byte piece, widened to 32 bytes).
  constexpr int kPieces = kFp8 ? 1 : 2;
  uint4 stage[kPieces];
  auto fetch = [&](int64_t base) {
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int piece = tid + u * 256;
      const int key = kFp8 ? (piece >> 3) : (piece >> 4);
      const int part = kFp8 ? (piece & 7) : (piece & 15);
      const int64_t row = base + key;
      if (row < a.k_rows) {
        const uint8_t* src = static_cast<const uint8_t*>(a.k_idx) +
                             row * (kFp8 ? kIxDim : 2 * kIxDim) + part * 16;
        stage[u] = *reinterpret_cast<const uint4*>(src);
      } else {
        stage[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int piece = tid + u * 256;
      if constexpr (kFp8) {
        const int key = piece >> 3, part = piece & 7;
        uint8_t* dst = &ktile[buf][key * kIxRowBytes + part * 32];
        const uint2 a0 = fp8x4_to_bf16x4(stage[u].x);
        const uint2 a1 = fp8x4_to_bf16x4(stage[u].y);
        const uint2 a2 = fp8x4_to_bf16x4(stage[u].z);
        const uint2 a3 = fp8x4_to_bf16x4(stage[u].w);
        *reinterpret_cast<uint4*>(dst) = make_uint4(a0.x, a0.y, a1.x, a1.y);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(a2.x, a2.y, a3.x, a3.y);
      } else {
        const int key = piece >> 4, part = piece & 15;
        *reinterpret_cast<uint4*>(&ktile[buf][key * kIxRowBytes + part * 16]) = stage[u];
      }
    }
  };

  fetch(t_first);
  for (int32_t t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int64_t base = t_first + static_cast<int64_t>(t) * kIxTileKeys;
    commit(buf);
    __syncthreads();
    if (t + 1 < n_tiles) fetch(base + kIxTileKeys);

    f32x16 acc[kIxQPerWave][kIxRowBlocks];
    bool act[kIxQPerWave];
#pragma unroll
    for (int s = 0; s < kIxQPerWave; ++s) {
      act[s] = my_lo[s] < base + kIxTileKeys && base < my_hi[s];
#pragma unroll
      for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[s][rb][i] = 0.f;
    }
    if (act[0] || act[1]) {
      const uint8_t* krow = &ktile[buf][(lane & 31) * kIxRowBytes + (lane >> 5) * 16];
#pragma unroll
      for (int ks = 0; ks < kIxKSteps; ++ks) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 32));
#pragma unroll
        for (int s = 0; s < kIxQPerWave; ++s) {
          if (!act[s]) continue;
#pragma unroll
          for (int rb = 0; rb < kIxRowBlocks; ++rb)
            acc[s][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s][rb][ks], b, acc[s][rb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int s = 0; s < kIxQPerWave; ++s) {
        if (!act[s]) continue;
        float v = head_sum(acc[s], wl[wave * kIxQPerWave + s], lane);
        const int64_t row = base + (lane & 31);
        if (lane < 32 && row >= my_lo[s] && row < my_hi[s]) {
          if constexpr (kFp8) v *= a.k_scale[row / kFp8BlockRows];
          a.scores[static_cast<int64_t>(my_j[s]) * a.score_stride + (row - my_lo[s])] = v;
        }
      }
    }
  }
}

// ----------------------------------------------------- decode, MFMA path
constexpr int kIxDecodeChunk = kIxWaves * 64;   // positions per workgroup

template <bool kFp8>
__global__ void __launch_bounds__(256)
indexer_paged_mfma_kernel(IndexerArgs a, int32_t n_chunks) {
  __shared__ float wl[kIxHeads];
  const int32_t j = blockIdx.x / n_chunks;
  const int32_t chunk = blockIdx.x - j * n_chunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (j >= a.n_q) return;
  const int32_t L = clamp_len(a, j);
  const int64_t pos0 = static_cast<int64_t>(chunk) * kIxDecodeChunk;
  if (pos0 >= L) return;
  if (tid < kIxHeads) wl[tid] = a.w[static_cast<int64_t>(j) * kIxHeads + tid];
  __syncthreads();
  const int64_t wpos = pos0 + wave * 64;
  if (wpos >= L) return;

  const int32_t req = a.q_req ? a.q_req[j] : 0;
  const int64_t kv0 = a.kv_start[j];
  const uint16_t* q0 = static_cast<const uint16_t*>(a.q_idx) +
                       static_cast<int64_t>(j) * kIxHeads * kIxDim;
  bf16x8 qa[kIxRowBlocks][kIxKSteps];
#pragma unroll
  for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
    for (int ks = 0; ks < kIxKSteps; ++ks) qa[rb][ks] = load_q_frag(q0, rb, ks, lane);

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t p = wpos + nb * 32 + (lane & 31);
    const int64_t row = p < L ? index_key_row(a, req, kv0 + p) : -1;
    bf16x8 kb[kIxKSteps];
#pragma unroll
    for (int ks = 0; ks < kIxKSteps; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row >= 0) {
        if constexpr (kFp8) {
          const uint2 c = *reinterpret_cast<const uint2*>(
              static_cast<const uint8_t*>(a.k_idx) + row * kIxDim + ks * 16 + (lane >> 5) * 8);
          const uint2 lo = fp8x4_to_bf16x4(c.x);
          const uint2 hi = fp8x4_to_bf16x4(c.y);
          v = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_idx) +
                                              row * kIxDim + ks * 16 + (lane >> 5) * 8);
        }
      }
      kb[ks] = __builtin_bit_cast(bf16x8, v);
    }
    f32x16 acc[kIxRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kIxKSteps; ++ks)
#pragma unroll
      for (int rb = 0; rb < kIxRowBlocks; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][ks], kb[ks], acc[rb], 0, 0, 0);
    float v = head_sum(acc, wl, lane);
    if (lane < 32 && p < L) {
      if (row < 0) {
        v = -INFINITY;
      } else if constexpr (kFp8) {
        v *= a.k_scale[row / kFp8BlockRows];
      }
      a.scores[static_cast<int64_t>(j) * a.score_stride + p] = v;
    }
  }
}

// ------------------------------------------------------------------ host
static constexpr int32_t kIxChunkKeys = 1024;

ds_status launch_indexer_scores(const IndexerArgs& a, hipStream_t s) {
  if (a.n_q == 0 || a.max_kv_len == 0) return DS_OK;
  if (a.q_dtype == DS_F32) {
    const size_t smem = sizeof(float) * (a.h_idx * a.d_idx + a.h_idx);
    dim3 grid(static_cast<unsigned>(ceil_div(a.max_kv_len, 256)), a.n_q);
    indexer_f32_kernel<<<grid, 256, smem, s>>>(a);
    return check_launch("indexer_scores (f32)");
  }
  const bool fp8 = a.k_dtype == DS_FP8_E4M3FN;
  if (a.page_table != nullptr) {
    const int32_t n_chunks = static_cast<int32_t>(ceil_div(a.max_kv_len, kIxDecodeChunk));
    const int64_t blocks = static_cast<int64_t>(a.n_q) * n_chunks;
    if (fp8) indexer_paged_mfma_kernel<true><<<blocks, 256, 0, s>>>(a, n_chunks);
    else indexer_paged_mfma_kernel<false><<<blocks, 256, 0, s>>>(a, n_chunks);
    return check_launch("indexer_scores (paged)");
  }
  const int32_t n_qblocks = static_cast<int32_t>(ceil_div(a.n_q, kIxQBlock));
  const int32_t n_chunks = static_cast<int32_t>(ceil_div(a.k_rows, kIxChunkKeys));
  const uint32_t grid = static_cast<uint32_t>(round_up(static_cast<int64_t>(n_qblocks) * n_chunks, 8));
  if (fp8)
    indexer_prefill_mfma_kernel<true><<<grid, 256, 0, s>>>(a, n_qblocks, n_chunks, kIxChunkKeys, grid);
  else
    indexer_prefill_mfma_kernel<false><<<grid, 256, 0, s>>>(a, n_qblocks, n_chunks, kIxChunkKeys, grid);
  return check_launch("indexer_scores (prefill)");
}

}  // namespace ds32cp
