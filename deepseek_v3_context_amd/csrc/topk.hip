// Step 4: per-query top-k of the indexer scores.
//
// Sources: "[RFC]: Parallel strategy for Deepseek v3.2 like models",
// comment thread (the indexer keeps, per query, the top-k KV entries of its
// history); "[DeepSeek v3.2] 上下文并行详解", section 2C (the top-k index
// transform maps selections onto the logically ordered KV).  Reading: the
// k largest scores, ties to the lower key position; rows with fewer than k
// causal keys select all of them and pad with -1.
//
// One workgroup per query row.  Scores are mapped to order-preserving
// 32-bit keys and the k-th largest key is found by four 8-bit radix passes
// (LDS histogram + one-wave suffix scan per pass).  Rows that fit are
// cached in LDS so the passes never return to HBM; longer rows stream from
// L2/HBM.  A final ordered pass (ballot + per-wave counts) writes the
// selected positions in ascending order: every key above the threshold and
// the lowest-position keys equal to it, so the selected set is exactly the
// tie-to-lower-position set and the output is deterministic.
#include "common.h"

namespace ds32cp {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int32_t kTkCacheKeys = 32768;   // 128 KiB of LDS

__device__ __forceinline__ int64_t topk_key_row(const TopkArgs& a, int32_t req,
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

__global__ void __launch_bounds__(kTkThreads)
topk_kernel(TopkArgs a, int32_t cache_keys) {
  extern __shared__ uint32_t cache[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit, sh_remaining;
  __shared__ uint32_t wave_eq[kTkWaves];

  const int32_t j = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int32_t L = a.kv_len[j];
  L = L < 0 ? 0 : (L > a.max_kv_len ? a.max_kv_len : L);
  const float* row_scores = a.scores + static_cast<int64_t>(j) * a.score_stride;
  int32_t* out_idx = a.topk_idx + static_cast<int64_t>(j) * a.topk;
  float* out_score = a.topk_score ? a.topk_score + static_cast<int64_t>(j) * a.topk : nullptr;
  const int32_t req = a.q_req ? a.q_req[j] : 0;
  const int64_t kv0 = a.kv_start[j];

  if (L <= a.topk) {  // every causal key is selected
    for (int32_t t = tid; t < a.topk; t += kTkThreads) {
      const bool take = t < L;
      out_idx[t] = take ? static_cast<int32_t>(topk_key_row(a, req, kv0 + t)) : -1;
      if (out_score) out_score[t] = take ? row_scores[t] : -INFINITY;
    }
    return;
  }

  const bool cached = L <= cache_keys;
  if (cached) {
    for (int32_t t = tid; t < L; t += kTkThreads) cache[t] = float_order_key(row_scores[t]);
  }
  auto key_at = [&](int32_t t) -> uint32_t {
    return cached ? cache[t] : float_order_key(row_scores[t]);
  };

  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(a.topk);
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTkThreads) hist[i] = 0;
    __syncthreads();
    for (int32_t t = tid; t < L; t += kTkThreads) {
      const uint32_t u = key_at(t);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 4l..4l+3; scan counts from the largest digit down
      uint32_t c[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) c[b] = hist[4 * lane + b];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = mine;  // sum over lanes >= this lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t other = __shfl_down(incl, off);
        if (lane + off < 64) incl += other;
      }
      uint32_t cum = incl - mine;   // keys in digits above this lane's four
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (cum < remaining && cum + c[b] >= remaining) {
          sh_digit = 4u * lane + b;
          sh_remaining = remaining - cum;
        }
        cum += c[b];
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining = sh_remaining;
    __syncthreads();
  }

  // prefix is now the k-th largest key; `remaining` copies of it are taken.
  // One ordered pass writes every selected position in ascending order:
  // keys above the threshold, and the first `remaining` keys equal to it.
  uint32_t taken = 0, eq_seen = 0;
  for (int32_t base = 0; base < L; base += kTkThreads) {
    const int32_t t = base + tid;
    const uint32_t u = t < L ? key_at(t) : 0u;
    const bool gt = t < L && u > prefix;
    const bool eq = t < L && u == prefix;
    const uint64_t ball_eq = __ballot(eq);
    // an equal key is taken when fewer than `remaining` equal keys precede it
    const uint32_t eq_rank_in_wave = static_cast<uint32_t>(__popcll(ball_eq & ((1ull << lane) - 1ull)));
    if (lane == 0) wave_eq[wave] = static_cast<uint32_t>(__popcll(ball_eq));
    __syncthreads();
    uint32_t eq_before = eq_seen;
    uint32_t eq_total = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t cnt = wave_eq[w];
      eq_before += w < wave ? cnt : 0u;
      eq_total += cnt;
    }
    const bool take = gt || (eq && eq_before + eq_rank_in_wave < remaining);
    const uint64_t ball_take = __ballot(take);
    __syncthreads();   // wave_eq is reused below
    if (lane == 0) wave_eq[wave] = static_cast<uint32_t>(__popcll(ball_take));
    __syncthreads();
    uint32_t take_before = taken, take_total = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t cnt = wave_eq[w];
      take_before += w < wave ? cnt : 0u;
      take_total += cnt;
    }
    if (take) {
      const uint32_t slot = take_before +
          static_cast<uint32_t>(__popcll(ball_take & ((1ull << lane) - 1ull)));
      if (slot < static_cast<uint32_t>(a.topk)) {
        out_idx[slot] = static_cast<int32_t>(topk_key_row(a, req, kv0 + t));
        if (out_score) out_score[slot] = order_key_to_float(u);
      }
    }
    taken += take_total;
    eq_seen += eq_total;
    __syncthreads();
    if (taken >= static_cast<uint32_t>(a.topk)) break;   // uniform: all threads agree
  }
}

ds_status launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_q == 0) return DS_OK;
  const int32_t cache_keys = a.max_kv_len < kTkCacheKeys ? a.max_kv_len : kTkCacheKeys;
  const size_t smem = sizeof(uint32_t) * static_cast<size_t>(cache_keys > 0 ? cache_keys : 1);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize,
                        static_cast<int>(sizeof(uint32_t) * kTkCacheKeys));
    attr_set = true;
  }
  topk_kernel<<<a.n_q, kTkThreads, smem, s>>>(a, cache_keys);
  return check_launch("topk_select");
}

}  // namespace ds32cp
