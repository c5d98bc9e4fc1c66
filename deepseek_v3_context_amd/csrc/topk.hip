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
// 32-bit keys.  In launches for long rows, rows of up to 65536 keys take
// the bitmap path: one read
// of the row from memory (16-bit keys cached in LDS, a 4096-bin histogram of
// the top 12 bits), a pass over the cache that records the keys above the
// threshold bin in a bitmap of positions, an exact resolution of the
// threshold bin's few keys, and one scan of the bitmap for the output.
// Other rows (and rows whose threshold bin is too crowded) take the general
// path: the k-th largest key is found by four 8-bit radix passes (per-wave
// LDS histograms + one-wave suffix scan per pass); rows that fit are cached
// in LDS so the passes never return to memory, longer rows are staged
// through LDS block by block on every pass, and a final ordered pass
// (block-wide scans) writes the selected positions.  Both write every key
// above the threshold and the lowest-position keys equal to it, in
// ascending position order, so the selected set is exactly the
// tie-to-lower-position set and the output is deterministic.
#include <mutex>

#include "common.h"

namespace ds32cp {

constexpr int kTkPer = 8;                 // consecutive keys per thread and step
constexpr int32_t kTkCacheKeys = 32768;   // 128 KiB of LDS
constexpr int32_t kTkSmallCacheKeys = 6144;   // 24 KiB: with 28 KiB of static LDS, three workgroups per CU (kMode 3)
// Bitmap path: bins of the first digit (the top 12 bits of the 32-bit
// key), the most threshold-bucket keys it resolves in LDS, and the longest
// row it takes (16-bit keys in the cache; positions fit in 16 bits).  Only
// the 1024-thread kernel (long rows) has it: the 512-thread one keeps its
// smaller LDS footprint, and with it two or three workgroups per CU.
constexpr int kTkBins = 4096;
constexpr int kTkCandMax = 2048;
constexpr int32_t kTkBitmapMaxLen = kTopkOnePassMaxLen;

// Physical KV row of logical position l (kv_start + key position) of
// request req, or -1.  Positions and kv_start are int32 by interface, so
// 0 <= l < 2^32 and the page division is an exact 32-bit one (a 64-bit
// division is a long instruction sequence).
__device__ __forceinline__ int64_t topk_key_row(const TopkArgs& a, int32_t req,
                                                int64_t l) {
  if (l < 0) return -1;
  if (a.page_table == nullptr) return l < a.k_rows ? l : -1;
  const uint32_t ps = static_cast<uint32_t>(a.page_size);
  const uint32_t pg = static_cast<uint32_t>(l) / ps;
  if (req < 0 || req >= a.n_req || pg >= static_cast<uint32_t>(a.max_pages)) return -1;
  const int32_t pid = a.page_table[static_cast<int64_t>(req) * a.max_pages + pg];
  const int64_t row = static_cast<int64_t>(pid) * ps + (static_cast<uint32_t>(l) - pg * ps);
  return (pid >= 0 && row < a.k_rows) ? row : -1;
}

// topk_key_row of kN positions kv0 + pos[i] at once, every page-table load
// issued before any is used; entries with use[i] false come out as -1.
template <int kN>
__device__ __forceinline__ void topk_key_rows(const TopkArgs& a, int32_t req, int64_t kv0,
                                              const int32_t (&pos)[kN], const bool (&use)[kN],
                                              int32_t (&row)[kN]) {
  if (a.page_table == nullptr) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int64_t l = kv0 + pos[i];
      row[i] = use[i] && l >= 0 && l < a.k_rows ? static_cast<int32_t>(l) : -1;
    }
    return;
  }
  const bool req_ok = req >= 0 && req < a.n_req;
  const int32_t* tab = a.page_table + static_cast<int64_t>(req_ok ? req : 0) * a.max_pages;
  const uint32_t ps = static_cast<uint32_t>(a.page_size);
  uint32_t pg[kN];
  int32_t pid[kN];
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int64_t l = kv0 + pos[i];
    pg[i] = l >= 0 ? static_cast<uint32_t>(l) / ps : 0xffffffffu;
  }
#pragma unroll
  for (int i = 0; i < kN; ++i)
    pid[i] = tab[use[i] && pg[i] < static_cast<uint32_t>(a.max_pages) ? pg[i] : 0u];
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int64_t l = kv0 + pos[i];
    const int64_t r = static_cast<int64_t>(pid[i]) * ps + (static_cast<uint32_t>(l) - pg[i] * ps);
    const bool ok = use[i] && req_ok && pg[i] < static_cast<uint32_t>(a.max_pages) &&
                    pid[i] >= 0 && r < a.k_rows;
    row[i] = ok ? static_cast<int32_t>(r) : -1;
  }
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

// Bitmap path of the single-workgroup selection (see topk_kernel).  Returns
// false, having written nothing, when the threshold bin holds more than
// kTkCandMax keys.  Uniform control flow: every thread takes every branch.
template <int kTkThreads, bool kCached>
__device__ bool bitmap_path(const TopkArgs& a, int32_t L, const float* row_scores,
                            int32_t* out_idx, float* out_score, int32_t req, int64_t kv0,
                            uint32_t* cache, int32_t c16_len, uint32_t* hw, uint16_t* cand_pos,
                            uint32_t* cand_key, uint32_t* wave_tot, uint32_t& sh_digit,
                            uint32_t& sh_remaining, uint32_t& sh_count, uint32_t& sh_ncand) {
  constexpr int kTkWaves = kTkThreads / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint16_t* c16 = reinterpret_cast<uint16_t*>(cache);
  const uint32_t k = static_cast<uint32_t>(a.topk);

  // The digit of `bins` bins (a power of two, a multiple of kTkThreads)
  // holding the `want`-th largest counted key: counts in hist[0..bins),
  // thread t owns bins [(n-1-t)*per, (n-t)*per) so that thread order is
  // descending bin order.  Sets sh_digit, sh_remaining (keys still wanted
  // from that bin) and sh_count (the bin's count).
  auto find_bin = [&](const uint32_t* hist, int bins, uint32_t want) {
    const int per = bins / kTkThreads;
    const int b0 = bins - per * (tid + 1);
    uint32_t c = 0;
    for (int i = 0; i < per; ++i) c += hist[b0 + i];
    uint32_t total;
    uint32_t cum = tk_block_scan<kTkWaves>(c, lane, wave, wave_tot, total);   // keys in higher bins
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t ci = hist[b0 + i];
      if (cum < want && cum + ci >= want) {
        sh_digit = static_cast<uint32_t>(b0 + i);
        sh_remaining = want - cum;
        sh_count = ci;
      }
      cum += ci;
    }
    __syncthreads();
  };

  // ---- pass A: the row from memory, 4 keys per thread and load
  for (int i = tid; i < kTkBins; i += kTkThreads) hw[i] = 0u;
  __syncthreads();
  const bool vec = (reinterpret_cast<uintptr_t>(row_scores) & 15u) == 0;
  // 16 loads of 16 bytes in flight per thread: a row of 65536 keys in one
  // round (this pass waits on memory, not on its arithmetic)
  constexpr int kU = kCached ? 16 : 8;
  for (int32_t r0 = 0; r0 < L; r0 += 4 * kTkThreads * kU) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t t = r0 + 4 * (u * kTkThreads + tid);
      if (vec && t + 4 <= L) {
        v[u] = *reinterpret_cast<const float4*>(row_scores + t);
      } else {
        v[u].x = t < L ? row_scores[t] : 0.f;
        v[u].y = t + 1 < L ? row_scores[t + 1] : 0.f;
        v[u].z = t + 2 < L ? row_scores[t + 2] : 0.f;
        v[u].w = t + 3 < L ? row_scores[t + 3] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t t = r0 + 4 * (u * kTkThreads + tid);
      if (t >= L) continue;
      const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t key[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) key[e] = float_order_key(f[e]);
      if (kCached || t + 4 <= c16_len) {
        if (t + 4 <= L) {
          *reinterpret_cast<uint2*>(c16 + t) =
              make_uint2((key[0] >> 16) | (key[1] & 0xffff0000u), (key[2] >> 16) | (key[3] & 0xffff0000u));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t + e < L) c16[t + e] = static_cast<uint16_t>(key[e] >> 16);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t + e < L) atomicAdd(&hw[key[e] >> 20], 1u);
    }
  }
  __syncthreads();
  find_bin(hw, kTkBins, k);
  const uint32_t T = sh_digit;
  uint32_t remaining = sh_remaining;   // keys still wanted from bin T
  const uint32_t n_t = sh_count;
  if (n_t > static_cast<uint32_t>(kTkCandMax)) return false;   // uniform

  // ---- pass B: bitmap of keys in bins above T, positions of bin T.  The
  // bitmap takes words [0, 2048) of hw (the histogram is consumed).
  uint32_t* bm = hw;
  uint32_t* aux = hw + 2048;   // radix histogram, then the tie bitmap
  const int32_t n_words = (L + 31) >> 5;
  if (tid == 0) sh_ncand = 0;
  __syncthreads();
  for (int32_t w0 = 0; w0 < n_words; w0 += kTkThreads) {
    const int32_t w = w0 + tid;
    uint32_t bits = 0, tbits = 0;
    if (w < n_words) {
      const int32_t p0 = w << 5;
      if (!kCached && p0 + 32 > c16_len) {
        // words past the row's cached head, again from memory (L2 or
        // HBM): 32 keys per word
        float4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int32_t t = p0 + 4 * q;
          if (vec && t + 4 <= L) {
            v[q] = *reinterpret_cast<const float4*>(row_scores + t);
          } else {
            v[q].x = t < L ? row_scores[t] : 0.f;
            v[q].y = t + 1 < L ? row_scores[t + 1] : 0.f;
            v[q].z = t + 2 < L ? row_scores[t + 2] : 0.f;
            v[q].w = t + 3 < L ? row_scores[t + 3] : 0.f;
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float f[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t t = p0 + 4 * q + e;
            const uint32_t b = float_order_key(f[e]) >> 20;
            bits |= (t < L && b > T ? 1u : 0u) << (4 * q + e);
            tbits |= (t < L && b == T ? 1u : 0u) << (4 * q + e);
          }
        }
      } else if (p0 + 32 <= L) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 x = *reinterpret_cast<const uint4*>(c16 + p0 + 8 * q);
          const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            const uint32_t b = ((wd[h >> 1] >> (16 * (h & 1))) & 0xffffu) >> 4;
            bits |= (b > T ? 1u : 0u) << (8 * q + h);
            tbits |= (b == T ? 1u : 0u) << (8 * q + h);
          }
        }
      } else {
        for (int e = 0; p0 + e < L; ++e) {
          const uint32_t b = static_cast<uint32_t>(c16[p0 + e]) >> 4;
          bits |= (b > T ? 1u : 0u) << e;
          tbits |= (b == T ? 1u : 0u) << e;
        }
      }
      bm[w] = bits;
    }
    // the bin's positions, appended wave by wave (their order is free)
    const uint32_t nt = static_cast<uint32_t>(__popc(tbits));
    uint32_t incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    uint32_t base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&sh_ncand, incl);
    base = __shfl(base, 63) + incl - nt;
    while (tbits) {
      const int e = __builtin_ctz(tbits);
      tbits &= tbits - 1u;
      if (base < static_cast<uint32_t>(kTkCandMax)) cand_pos[base] = static_cast<uint16_t>((w << 5) + e);
      ++base;
    }
  }
  __syncthreads();
  const int32_t n_c = static_cast<int32_t>(n_t);   // == sh_ncand: every key was counted once

  // ---- the k-th largest key among bin T: full keys, two 10-bit passes
  for (int32_t i = tid; i < n_c; i += kTkThreads)
    cand_key[i] = float_order_key(row_scores[cand_pos[i]]);
  uint32_t prefix = T << 20, mask = 0xfff00000u;
  for (int shift = 10; shift >= 0; shift -= 10) {
    for (int i = tid; i < 1024; i += kTkThreads) aux[i] = 0u;
    __syncthreads();
    for (int32_t i = tid; i < n_c; i += kTkThreads) {
      const uint32_t u = cand_key[i];
      if ((u & mask) == prefix) atomicAdd(&aux[(u >> shift) & 1023u], 1u);
    }
    __syncthreads();
    find_bin(aux, 1024, remaining);
    prefix |= sh_digit << shift;
    mask |= 1023u << shift;
    remaining = sh_remaining;
    __syncthreads();   // sh_* read by all before the next pass writes them
  }
  const uint32_t thr = prefix;           // the k-th largest key of the row
  const uint32_t n_eq = sh_count;        // keys equal to it
  const bool all_eq = remaining == n_eq; // every one of them is taken

  // ---- keys of bin T above the threshold join the bitmap; equal keys go
  // to the tie bitmap (aux), unless all of them are taken
  for (int32_t i = tid; i < n_words; i += kTkThreads) aux[i] = 0u;
  __syncthreads();
  for (int32_t i = tid; i < n_c; i += kTkThreads) {
    const uint32_t u = cand_key[i];
    const uint32_t p = cand_pos[i];
    if (u > thr || (u == thr && all_eq)) atomicOr(&bm[p >> 5], 1u << (p & 31u));
    else if (u == thr) atomicOr(&aux[p >> 5], 1u << (p & 31u));
  }
  __syncthreads();
  // thread t covers words [wpt*t, wpt*t + wpt): thread order is position order
  constexpr int kWpt = 2048 / kTkThreads;
  if (!all_eq) {   // uniform: the lowest `remaining` tied positions
    uint32_t tw[kWpt], c = 0;
#pragma unroll
    for (int q = 0; q < kWpt; ++q) {
      const int32_t w = kWpt * tid + q;
      tw[q] = w < n_words ? aux[w] : 0u;
      c += static_cast<uint32_t>(__popc(tw[q]));
    }
    uint32_t total;
    uint32_t r = tk_block_scan<kTkWaves>(c, lane, wave, wave_tot, total);
#pragma unroll
    for (int q = 0; q < kWpt; ++q) {
      uint32_t take = 0, x = tw[q];
      while (x) {
        const uint32_t bit = x & (0u - x);
        x ^= bit;
        if (r < remaining) take |= bit;
        ++r;
      }
      if (take) atomicOr(&bm[kWpt * tid + q], take);
    }
    __syncthreads();
  }

  // ---- ascending positions of the selected keys (exactly k of them),
  // ranked by one block scan into LDS (the candidate keys are consumed),
  // then mapped to rows and written out with coalesced stores
  uint32_t sw[kWpt], c = 0;
#pragma unroll
  for (int q = 0; q < kWpt; ++q) {
    const int32_t w = kWpt * tid + q;
    sw[q] = w < n_words ? bm[w] : 0u;
    c += static_cast<uint32_t>(__popc(sw[q]));
  }
  uint32_t total;
  uint32_t slot = tk_block_scan<kTkWaves>(c, lane, wave, wave_tot, total);
  uint32_t* sel = cand_key;
#pragma unroll
  for (int q = 0; q < kWpt; ++q) {
    uint32_t x = sw[q];
    while (x) {
      const int e = __builtin_ctz(x);
      x &= x - 1u;
      if (slot < k) sel[slot] = static_cast<uint32_t>(((kWpt * tid + q) << 5) + e);
      ++slot;
    }
  }
  __syncthreads();
  // every slot of the thread at once: page-table and score loads in flight
  // together
  constexpr int kOut = kTopkMax / kTkThreads;
  int32_t pos[kOut], row[kOut];
  bool use[kOut];
  float sc[kOut];
#pragma unroll
  for (int q = 0; q < kOut; ++q) {
    const uint32_t i = static_cast<uint32_t>(tid + q * kTkThreads);
    use[q] = i < k;
    pos[q] = use[q] ? static_cast<int32_t>(sel[i]) : 0;
  }
  topk_key_rows<kOut>(a, req, kv0, pos, use, row);
#pragma unroll
  for (int q = 0; q < kOut; ++q) sc[q] = out_score && use[q] ? row_scores[pos[q]] : 0.f;
#pragma unroll
  for (int q = 0; q < kOut; ++q) {
    if (!use[q]) continue;
    const int32_t i = tid + q * kTkThreads;
    out_idx[i] = row[q];
    if (out_score) out_score[i] = order_key_to_float(float_order_key(sc[q]));
  }
  return true;
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
// kMode 3: kMode 0 for launches of many rows of more than 4096 keys (512
//   threads, three workgroups per CU): the bitmap path reads the row twice
//   from memory, except its first keys, whose top 16 bits stay in the small
//   block cache between the two passes; the general path works on that
//   block cache.
template <int kTkThreads, int kMode>
__device__ __forceinline__ void topk_body(const TopkArgs& a, int32_t cache_keys) {
  constexpr int kTkWaves = kTkThreads / kWave;
  // the bitmap path: with the row's top 16 bits cached in LDS (kMode 0,
  // 1024 threads), or reading all but its head twice from memory (kMode 3: 512
  // threads and a small LDS footprint, so that three workgroups share a CU
  // and one's memory passes run under the others' LDS and ALU work)
  constexpr bool kBitmap = (kMode == 0 && kTkThreads == 1024) || kMode == 3;
  static_assert(kMode != 3 || kTkThreads == 512, "kMode 3 is the 512-thread kernel");
  extern __shared__ __align__(16) uint32_t cache[];
  // one 256-bin histogram per wave (less contention); the bitmap path uses
  // the same words as one 4096-bin histogram, then as its bitmaps
  constexpr int kHistWords = kBitmap && kTkBins > kTkWaves * 256 ? kTkBins : kTkWaves * 256;
  __shared__ uint32_t hist_words[kHistWords];
  uint32_t (*hist)[256] = reinterpret_cast<uint32_t (*)[256]>(hist_words);
  __shared__ uint32_t sh_digit, sh_remaining, sh_count, sh_ncand;
  __shared__ uint32_t wave_tot[kTkWaves];
  __shared__ int32_t sel_t[kTopkMax];        // selected elements in output order (kMode 0, 2)
  __shared__ uint16_t cand_pos[kBitmap ? kTkCandMax : 1];   // bitmap path: bucket positions

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

  // ---- bitmap path (rows of up to 65536 keys, 1024-thread kernel).  The row is read from
  // memory once: every key's top 16 bits go to LDS and its top 12 bits are
  // counted.  The bin holding the k-th largest key (the threshold bin) then
  // splits the row: keys in higher bins are selected, and a pass over the
  // cached keys records them in a bitmap of positions and lists the
  // positions of the threshold bin.  Those (few) keys are read again in
  // full and the k-th largest key is found among them by two 10-bit radix
  // passes; keys above it join the bitmap, and of the keys equal to it the
  // lowest positions are taken (their own bitmap, ranked by a scan).  One
  // scan over the bitmap writes the selected positions in ascending order.
  // When the threshold bin holds more than kTkCandMax keys (scores sharing
  // their top 12 bits en masse) the general radix passes below take over.
  if constexpr (kBitmap) {
    if ((kMode == 3 || L <= 2 * cache_keys) && L <= kTkBitmapMaxLen &&
        bitmap_path<kTkThreads, kMode == 0>(a, L, row_scores, out_idx,
        out_score, req, kv0, cache,
        kMode == 0 ? L : (L < 2 * cache_keys ? L : 2 * cache_keys) & ~31,
        hist_words, cand_pos, reinterpret_cast<uint32_t*>(sel_t),
        wave_tot, sh_digit, sh_remaining, sh_count, sh_ncand)) {
      return;
    }
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
    if ((kMode == 0 || kMode == 3) && shift == 24 && !cached && sh_count <= static_cast<uint32_t>(cache_keys)) {
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

template <int kTkThreads, int kMode>
__global__ void __launch_bounds__(kTkThreads) topk_kernel(TopkArgs a, int32_t cache_keys) {
  topk_body<kTkThreads, kMode>(a, cache_keys);
}

// kMode 3: three workgroups of 512 threads per CU, so at most 80 VGPRs
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(6)))
topk_rows_kernel(TopkArgs a, int32_t cache_keys) {
  topk_body<512, 3>(a, cache_keys);
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
  if (a.max_kv_len > 4096 && a.max_kv_len <= kTkBitmapMaxLen && a.n_q >= 2 * device_cu_count()) {
    // many rows of more than 4096 keys: three rows per CU, the memory passes
    // of one under the LDS and ALU work of the others; a small block cache
    // for the rare rows that leave the bitmap path
    const int32_t ck = a.max_kv_len < kTkSmallCacheKeys ? a.max_kv_len : kTkSmallCacheKeys;
    topk_rows_kernel<<<a.n_q, 512, sizeof(uint32_t) * ck, s>>>(a, ck);
  } else if (a.max_kv_len > 16384) {
    // few long rows: more waves per row to keep more keys in flight
    topk_kernel<1024, 0><<<a.n_q, 1024, smem, s>>>(a, cache_keys);
  } else {
    topk_kernel<512, 0><<<a.n_q, 512, smem, s>>>(a, cache_keys);
  }
  return check_launch("topk_select");
}

}  // namespace ds32cp
