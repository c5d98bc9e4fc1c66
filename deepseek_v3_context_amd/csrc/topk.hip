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
// (per-wave LDS histograms + one-wave suffix scan per pass).  Rows that fit
// are cached in LDS so the passes never return to memory; longer rows are
// staged through LDS block by block on every pass.  A final ordered pass
// (block-wide scans) writes the selected positions in ascending order:
// every key above the threshold and the lowest-position keys equal to it,
// so the selected set is exactly the tie-to-lower-position set and the
// output is deterministic.
#include <mutex>

#include "common.h"

namespace ds32cp {

constexpr int kTkPer = 8;                 // consecutive keys per thread and step
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

// Exclusive prefix sum of one count per thread over the workgroup, in
// thread order, plus the total.  Uses wave_tot (one slot per wave); two
// barriers.
template <int kTkWaves>
__device__ __forceinline__ uint32_t tk_block_scan(uint32_t v, int lane, int wave,
                                                  uint32_t* wave_tot, uint32_t& total) {
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint32_t c = wave_tot[w];
    before += w < wave ? c : 0u;
    tot += c;
  }
  __syncthreads();   // wave_tot may be reused right after
  total = tot;
  return before + incl - v;
}

// kMode 0: one workgroup selects a whole row.
// kMode 1 (two-phase, first phase): workgroup (row, s) selects the top-k of
//   positions [s*seg_len, (s+1)*seg_len) of its row and writes them (score
//   and position), in position order and padded to k entries (score -inf,
//   position -1), to the row's candidate list.  The row's top-k is a
//   subset of the union of its segments' top-k (ties included: a segment
//   keeps its lowest positions among equal scores), so nothing is lost.
// kMode 2 (second phase): one workgroup selects the row's top-k from its
//   n_seg*k candidates, which are in position order; padding scores are
//   -inf, below every finite score (a key scored -inf is an unmapped one,
//   whose row is -1 like a padding entry's, so ties there change nothing).
template <int kTkThreads, int kMode>
__global__ void __launch_bounds__(kTkThreads)
topk_kernel(TopkArgs a, int32_t cache_keys) {
  constexpr int kTkWaves = kTkThreads / kWave;
  extern __shared__ __align__(16) uint32_t cache[];
  __shared__ uint32_t hist[kTkWaves][256];   // one histogram per wave (less contention)
  __shared__ uint32_t sh_digit, sh_remaining, sh_count, sh_ncand;
  __shared__ uint32_t wave_tot[kTkWaves];
  __shared__ int32_t sel_t[kTopkMax];        // selected elements in output order (kMode 0, 2)

  const int32_t j = kMode == 1 ? static_cast<int32_t>(blockIdx.x / a.n_seg) : blockIdx.x;
  const int32_t seg = kMode == 1 ? static_cast<int32_t>(blockIdx.x % a.n_seg) : 0;
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
  const int64_t cbase = static_cast<int64_t>(j) * a.n_seg * a.topk;   // row's candidates
  int32_t pos0 = 0;   // logical position of element 0 (kMode 1)
  if constexpr (kMode == 1) {
    pos0 = seg * a.seg_len;
    L = L - pos0 < a.seg_len ? L - pos0 : a.seg_len;
    L = L < 0 ? 0 : L;
    row_scores += pos0;
  } else if constexpr (kMode == 2) {
    row_scores = a.cand_score + cbase;
    if (L > a.topk) L = a.n_seg * a.topk;
  }
  // What element t contributes: in the first phase of the two-phase
  // selection its logical position (the candidates keep position order,
  // and only the final k are mapped); otherwise its output row, the
  // physical KV row of its position (-1 when unmapped or padding).
  auto row_of = [&](int32_t t) -> int32_t {
    if constexpr (kMode == 1) {
      return pos0 + t;
    } else if constexpr (kMode == 2) {
      const int32_t p = a.cand_pos[cbase + t];
      return p >= 0 ? static_cast<int32_t>(topk_key_row(a, req, kv0 + p)) : -1;
    } else {
      return static_cast<int32_t>(topk_key_row(a, req, kv0 + t));
    }
  };
  // the slot-th selected element (position order) contributes `v`
  auto emit = [&](uint32_t slot, int32_t v, float score) {
    if constexpr (kMode == 1) {
      const int64_t c = cbase + static_cast<int64_t>(seg) * a.topk + slot;
      a.cand_score[c] = score;
      a.cand_pos[c] = v;
    } else {
      out_idx[slot] = v;
      if (out_score) out_score[slot] = score;
    }
  };

  if (L <= a.topk) {  // every key is selected
    for (int32_t t = tid; t < a.topk; t += kTkThreads) {
      if (t < L) {
        emit(t, row_of(t), row_scores[t]);
      } else if constexpr (kMode == 1) {
        const int64_t c = cbase + static_cast<int64_t>(seg) * a.topk + t;
        a.cand_score[c] = -INFINITY;
        a.cand_pos[c] = -1;
      } else {
        out_idx[t] = -1;
        if (out_score) out_score[t] = -INFINITY;
      }
    }
    return;
  }

  // The row is processed in blocks of cache_keys keys staged in LDS as
  // order-preserving keys (one block, loaded once, when the row fits).  A
  // block load keeps many loads in flight per thread, and every pass over
  // a block handles kTkPer consecutive keys per thread per step, so that
  // neither memory nor LDS latency is paid per key.
  const bool cached = L <= cache_keys;
  auto block_len = [&](int32_t b0) { return L - b0 < cache_keys ? L - b0 : cache_keys; };
  auto load_block = [&](int32_t b0) {
    const int32_t n = block_len(b0);
    constexpr int kU = 16;
    for (int32_t r0 = 0; r0 < n; r0 += kU * kTkThreads) {
      float v[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int32_t t = r0 + k * kTkThreads + tid;
        v[k] = t < n ? row_scores[b0 + t] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int32_t t = r0 + k * kTkThreads + tid;
        if (t < n) cache[t] = float_order_key(v[k]);
      }
    }
    __syncthreads();
  };
  // keys t0 .. t0+kTkPer-1 of the staged block (past its end: 0, and
  // masked out by the callers)
  auto read_keys = [&](int32_t t0, int32_t n, uint32_t (&u)[kTkPer]) {
    if (t0 + kTkPer <= n) {
      const uint4 x = *reinterpret_cast<const uint4*>(&cache[t0]);
      const uint4 y = *reinterpret_cast<const uint4*>(&cache[t0 + 4]);
      u[0] = x.x; u[1] = x.y; u[2] = x.z; u[3] = x.w;
      u[4] = y.x; u[5] = y.y; u[6] = y.z; u[7] = y.w;
    } else {
#pragma unroll
      for (int k = 0; k < kTkPer; ++k) u[k] = t0 + k < n ? cache[t0 + k] : 0u;
    }
  };
  if (cached) load_block(0);

  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(a.topk);
  // Histogram of digit `shift` of the keys that match the prefix so far,
  // over keys 0..n-1 of the staged block.
  auto count_keys = [&](int32_t n, int shift) {
    for (int32_t t0 = tid * kTkPer; t0 < n; t0 += kTkThreads * kTkPer) {
      uint32_t u[kTkPer];
      read_keys(t0, n, u);
#pragma unroll
      for (int k = 0; k < kTkPer; ++k) {
        const bool in = t0 + k < n && (u[k] & mask) == prefix;
        const uint32_t d = (u[k] >> shift) & 255u;
        // Scores of a row often share their top bits: lanes of the wave
        // with the digit of the first active lane are counted with one add.
        const uint64_t act = __ballot(in);
        if (act == 0ull) continue;
        const int first = static_cast<int>(__builtin_ctzll(act));
        const uint32_t d0 = __builtin_amdgcn_readlane(d, first);
        const uint64_t same = __ballot(in && d == d0);
        if (lane == first) atomicAdd(&hist[wave][d0], static_cast<uint32_t>(__popcll(same)));
        if (in && d != d0) atomicAdd(&hist[wave][d], 1u);
      }
    }
  };
  // Rows longer than the cache: after the first pass only the keys in the
  // threshold's top-byte bucket matter to the next three, so when they fit
  // they are compacted into the cache once (one more read of the row) and
  // the later passes count them there instead of reading the row again.
  bool cand = false;
  int32_t n_cand = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kTkWaves * 256; i += kTkThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    if (cand) {
      count_keys(n_cand, shift);
    } else {
      for (int32_t b0 = 0; b0 < L; b0 += cache_keys) {
        if (!cached) {
          __syncthreads();   // the previous block is fully counted
          load_block(b0);
        }
        count_keys(block_len(b0), shift);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 4l..4l+3; scan counts from the largest digit down
      uint32_t c[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t v = 0;
#pragma unroll
        for (int w = 0; w < kTkWaves; ++w) v += hist[w][4 * lane + b];
        c[b] = v;
      }
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
          sh_count = c[b];
        }
        cum += c[b];
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining = sh_remaining;
    __syncthreads();
    if (kMode == 0 && shift == 24 && !cached && sh_count <= static_cast<uint32_t>(cache_keys)) {
      // uniform: every thread read the same sh_count
      if (tid == 0) sh_ncand = 0;
      __syncthreads();   // (the cache's last staged block is fully counted)
      constexpr int kU = 16;
      for (int32_t r0 = 0; r0 < L; r0 += kU * kTkThreads) {
        float v[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
          const int32_t t = r0 + k * kTkThreads + tid;
          v[k] = t < L ? row_scores[t] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
          const int32_t t = r0 + k * kTkThreads + tid;
          const uint32_t u = float_order_key(v[k]);
          const bool m = t < L && (u & mask) == prefix;
          const uint64_t bm = __ballot(m);
          if (bm == 0ull) continue;
          uint32_t base = 0;
          if (lane == 0) base = atomicAdd(&sh_ncand, static_cast<uint32_t>(__popcll(bm)));
          base = __shfl(base, 0);
          const uint32_t slot = base + static_cast<uint32_t>(__popcll(bm & ((1ull << lane) - 1ull)));
          if (m && slot < static_cast<uint32_t>(cache_keys)) cache[slot] = u;
        }
      }
      __syncthreads();
      n_cand = static_cast<int32_t>(sh_ncand < static_cast<uint32_t>(cache_keys) ? sh_ncand
                                                                           : static_cast<uint32_t>(cache_keys));
      cand = true;
      __syncthreads();   // sh_ncand read by all before any later write
    }
  }

  // prefix is now the k-th largest key; `remaining` copies of it are taken.
  // One ordered pass writes every selected position in ascending order:
  // keys above the threshold, and the first `remaining` keys equal to it.
  // Thread t covers kTkPer consecutive positions of each step; two block
  // scans (equal keys, then taken keys) give every key its rank.
  uint32_t taken = 0, eq_seen = 0;
  for (int32_t b0 = 0; b0 < L && taken < static_cast<uint32_t>(a.topk); b0 += cache_keys) {
    if (!cached) {
      __syncthreads();
      load_block(b0);
    }
    const int32_t n = block_len(b0);
    for (int32_t s0 = 0; s0 < n; s0 += kTkThreads * kTkPer) {
      const int32_t t0 = s0 + tid * kTkPer;
      uint32_t u[kTkPer];
      read_keys(t0, n, u);
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int k = 0; k < kTkPer; ++k) {
        const bool v = t0 + k < n;
        gt |= (v && u[k] > prefix) ? 1u << k : 0u;
        eq |= (v && u[k] == prefix) ? 1u << k : 0u;
      }
      uint32_t eq_total;
      const uint32_t eq_before = eq_seen + tk_block_scan<kTkWaves>(__popc(eq), lane, wave, wave_tot, eq_total);
      // equal keys are taken while fewer than `remaining` precede them
      uint32_t take = gt;
      uint32_t r = eq_before;
#pragma unroll
      for (int k = 0; k < kTkPer; ++k) {
        if ((eq >> k) & 1u) {
          if (r < remaining) take |= 1u << k;
          ++r;
        }
      }
      uint32_t take_total;
      uint32_t slot = taken + tk_block_scan<kTkWaves>(__popc(take), lane, wave, wave_tot, take_total);
#pragma unroll
      for (int k = 0; k < kTkPer; ++k) {
        if ((take >> k) & 1u) {
          if (slot < static_cast<uint32_t>(a.topk)) {
            if constexpr (kMode == 1) emit(slot, row_of(b0 + t0 + k), order_key_to_float(u[k]));
            else sel_t[slot] = b0 + t0 + k;
          }
          ++slot;
        }
      }
      taken += take_total;
      eq_seen += eq_total;
      if (taken >= static_cast<uint32_t>(a.topk)) break;   // uniform: all threads agree
    }
  }
  if constexpr (kMode != 1) {
    // map the selected elements to rows with every lookup in flight at
    // once (a lookup may be two dependent loads: candidate position, then
    // page table)
    __syncthreads();
    for (int32_t s = tid; s < a.topk; s += kTkThreads) {
      const int32_t t = sel_t[s];
      emit(s, row_of(t), order_key_to_float(float_order_key(row_scores[t])));
    }
  }
}

template <int kThreads, int kMode>
static void topk_set_smem() {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel<kThreads, kMode>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(sizeof(uint32_t) * kTkCacheKeys));
}

ds_status launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_q == 0) return DS_OK;
  // the kernels' dynamic LDS limit, raised once per device (thread-safe)
  static std::once_flag attr_once[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DS_ERR_HIP, "topk_select: no current HIP device");
  std::call_once(attr_once[dev], [] {
    topk_set_smem<512, 0>();
    topk_set_smem<1024, 0>();
    topk_set_smem<512, 1>();
    topk_set_smem<1024, 2>();
  });
  if (a.cand_score != nullptr) {
    // two phases: segments of kTopkSegLen positions (cached in LDS), then
    // the candidates of each row (n_seg * topk, cached in LDS)
    const size_t smem1 = sizeof(uint32_t) * kTopkSegLen;
    topk_kernel<512, 1><<<a.n_q * a.n_seg, 512, smem1, s>>>(a, kTopkSegLen);
    ds_status st = check_launch("topk_select (segments)");
    if (st != DS_OK) return st;
    const int32_t nc = a.n_seg * a.topk;
    const int32_t cache2 = nc < kTkCacheKeys ? nc : kTkCacheKeys;
    topk_kernel<1024, 2><<<a.n_q, 1024, sizeof(uint32_t) * cache2, s>>>(a, cache2);
    return check_launch("topk_select (candidates)");
  }
  const int32_t cache_keys = a.max_kv_len < kTkCacheKeys ? a.max_kv_len : kTkCacheKeys;
  const size_t smem = sizeof(uint32_t) * static_cast<size_t>(cache_keys > 0 ? cache_keys : 1);
  // long rows: more waves per row to keep more keys in flight
  if (a.max_kv_len > 16384) topk_kernel<1024, 0><<<a.n_q, 1024, smem, s>>>(a, cache_keys);
  else topk_kernel<512, 0><<<a.n_q, 512, smem, s>>>(a, cache_keys);
  return check_launch("topk_select");
}

}  // namespace ds32cp
