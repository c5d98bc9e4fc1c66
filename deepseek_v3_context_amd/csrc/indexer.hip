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
//   * prefill: a workgroup of 8 waves owns 8 consecutive queries (one per
//     wave, A fragments and head weights in registers for the whole chunk)
//     and a chunk of absolute key rows; key tiles (128 bf16 or 256 fp8
//     rows) are gathered into LDS by DMA, double-buffered, and shared by
//     the 8 waves.  Queries of one workgroup may belong to different
//     requests: each masks its own causal range on write.
//   * decode: keys are paged per request; units of 32 positions are split
//     evenly over the resident waves, and each key row is read from HBM
//     exactly once (bf16 rows through a per-wave LDS transpose).
// fp8 keys are widened to bf16 exactly; the per-block scale is positive
// and multiplies the whole score of its key (ReLU commutes with a
// positive factor), so it is applied once per key after the head sum.
#include <type_traits>

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

// ReLU as one integer max of the bit pattern: a float with the sign bit set
// (negative, or -0) is a negative int and becomes +0, any other is kept.
// Exact for every non-NaN input (the MFMA results are finite); fmaxf would
// first quiet a possible signalling NaN with one more instruction per
// element, a third of the head-sum epilogue.
__device__ __forceinline__ float relu_raw(float x) {
  const int32_t b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// ------------------------------------------------------- MFMA constants
constexpr int kIxHeads = 64;
constexpr int kIxDim = 128;
constexpr int kIxKSteps = kIxDim / 16;        // K = 16 per MFMA
constexpr int kIxRowBlocks = kIxHeads / 32;   // M = 32 per MFMA
constexpr int kIxWaves = 4;                  // decode kernel: waves per workgroup

// A fragment of v_mfma_f32_32x32x16_bf16 for heads [32*rb, 32*rb+32) and
// dims [16*ks, 16*ks+16): lane l holds head 32*rb + l%32, dims
// 16*ks + 8*(l/32) + 0..7 (16 contiguous bytes).
__device__ __forceinline__ bf16x8 load_q_frag(const uint16_t* q_row0, int rb, int ks,
                                              int lane) {
  const uint16_t* p = q_row0 + (rb * 32 + (lane & 31)) * kIxDim + ks * 16 + (lane >> 5) * 8;
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// Weighted ReLU head-sum of one 64-head x 32-key accumulator pair (decode
// kernel).  Output element i of lane l sits at head 8*(i/4) + 4*(l/32) +
// i%4 (+32*rb), key l%32; after the cross-half swap every lane holds its
// key's full sum.
__device__ __forceinline__ float head_sum(const f32x16 (&acc)[kIxRowBlocks],
                                          const float* w_heads, int lane) {
  float v = 0.f;
#pragma unroll
  for (int rb = 0; rb < kIxRowBlocks; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = rb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      v = fmaf(w_heads[h], relu_raw(acc[rb][i]), v);
    }
  }
  v += __shfl_xor(v, 32);
  return v;
}

// --------------------------------------------- prefill: key tiles in LDS
// A workgroup of 8 waves works on 8 consecutive queries at a time (one per
// wave: A fragments in 64 VGPRs, the 64 head weights of the query in 32
// VGPRs).  Key tiles (128 bf16 or 256 fp8 rows) are gathered straight into
// LDS with global_load_lds_dwordx4 (no VGPRs), double-buffered so that the
// gather of the next tile overlaps the MFMAs of the current one; every wave
// reads the shared tile's B fragments from LDS.  Two waves per SIMD.
constexpr int kIxPWaves = 8;                       // waves (queries) per workgroup
constexpr int kIxPHalf = 64;                       // keys per MFMA pass (two 32-key blocks)
constexpr int kIxTileFp8 = 256, kIxTileBf16 = 128; // keys per tile
template <bool kFp8>
struct IxTile {
  // keys per tile (256 fp8 rows or 128 bf16 rows: about 36 KB of LDS)
  static constexpr int kTile = kFp8 ? kIxTileFp8 : kIxTileBf16;
  static constexpr int kRowBytes = kFp8 ? kIxDim : 2 * kIxDim;   // 128 / 256
  static constexpr int kRowShift = kFp8 ? 7 : 8;
  static constexpr int kLdsRow = kRowBytes + 16;                  // padded
  static constexpr int kChunksPerRow = kLdsRow / 16;              // 9 / 17
  static constexpr int kChunks = kTile * kChunksPerRow;           // 2304 / 2176
  static constexpr int kInst = kChunks / kWave;                   // 36 / 34
  static constexpr int kBytes = kInst * kWave * 16;               // LDS bytes per buffer
  static constexpr int kPer = (kInst + kIxPWaves - 1) / kIxPWaves; // DMA slots per wave: 5 / 5
  // instruction of slot i of a wave; past the last one, a repeat of the
  // wave's previous instruction (identical bytes to the same place)
  static __device__ __forceinline__ int inst(int wave, int i) {
    const int m = wave + i * kIxPWaves;
    return m < kInst ? m : m - kIxPWaves;
  }
};

constexpr int kIxBufBytes = IxTile<true>::kBytes > IxTile<false>::kBytes ? IxTile<true>::kBytes
                                                                         : IxTile<false>::kBytes;
__shared__ __align__(16) uint8_t g_ix_buf0[kIxBufBytes];
__shared__ __align__(16) uint8_t g_ix_buf1[kIxBufBytes];

template <int B>
__device__ __forceinline__ uint8_t* ix_buf() {
  return B ? g_ix_buf1 : g_ix_buf0;
}

// Byte offset, within a tile's key rows, of the 16 bytes each lane of slot
// i gathers (padding chunks re-read the row's last chunk).  Loop-invariant:
// computed once per wave.
template <bool kFp8>
struct IxSlots {
  using TL = IxTile<kFp8>;
  uint32_t off[TL::kPer];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < TL::kPer; ++i) {
      const int P = TL::inst(wave, i) * kWave + lane;
      const int r = P / TL::kChunksPerRow;
      const int c = P - r * TL::kChunksPerRow;
      const int cc = c < TL::kRowBytes / 16 ? c : TL::kRowBytes / 16 - 1;
      off[i] = static_cast<uint32_t>(r * TL::kRowBytes + cc * 16);
    }
  }
};

// Gathers key rows [base, base + 128) into buffer B: one DMA instruction per
// slot, SGPR base + the slot's constant offsets.  Rows at or past k_rows
// (the last tile of the key set) read the tile's first row instead; their
// scores are never stored.  The instructions are not visible to the
// compiler: the kernel waits for them itself before the tile barrier.
template <int B, bool kFp8>
__device__ __forceinline__ void ix_issue_tile(const uint8_t* keys, int64_t k_rows, int64_t base,
                                              const IxSlots<kFp8>& sl, int wave) {
  using TL = IxTile<kFp8>;
  const uint8_t* src = keys + base * TL::kRowBytes;
  const uint32_t lds = static_cast<uint32_t>(
      (size_t)((__attribute__((address_space(3))) uint8_t*)ix_buf<B>()));
  const bool full = base + TL::kTile <= k_rows;
  const uint32_t rows_valid = static_cast<uint32_t>(k_rows - base);
#pragma unroll
  for (int i = 0; i < TL::kPer; ++i) {
    uint32_t o = sl.off[i];
    if (!full) o = (o >> TL::kRowShift) < rows_valid ? o : (o & (TL::kRowBytes - 1));
    const uint32_t m0 = lds + static_cast<uint32_t>(TL::inst(wave, i) * kWave * 16);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(o), "s"(src), "s"(m0)
                 : "memory", "m0");
  }
}

// B fragment of v_mfma_f32_32x32x16_bf16 for key column (lane & 31) of the
// tile block `nb` and dims 16*ks + 8*(lane/32) + 0..7.
template <bool kFp8>
__device__ __forceinline__ bf16x8 ix_bfrag(const uint8_t* tile, int nb, int ks, int lane) {
  using TL = IxTile<kFp8>;
  const uint8_t* row = tile + (nb * 32 + (lane & 31)) * TL::kLdsRow;
  if constexpr (kFp8) {
    const uint2 c = *reinterpret_cast<const uint2*>(row + ks * 16 + (lane >> 5) * 8);
    const uint2 lo = fp8x4_to_bf16x4(c.x);
    const uint2 hi = fp8x4_to_bf16x4(c.y);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  } else {
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const uint4*>(row + ks * 32 + (lane >> 5) * 16));
  }
}

// ----------------------------------------------------- decode, MFMA path
// Work unit: 32 consecutive positions of one query (one MFMA N block).  The
// units of all queries, in query order, are split evenly over the resident
// waves (about two workgroups per CU), so every wave streams the same number
// of key rows whatever the mix of context lengths.  A wave walks its units
// query by query: the query's A fragments (64 VGPRs) and the 32 head
// weights its lanes reduce are loaded once per query, and the key fragments
// of the next unit are in flight while the current one runs its MFMAs.
// Physical rows are resolved through the page table one unit further
// ahead.  Every key row is read from HBM exactly once.
constexpr int kIxDUnit = 32;

__device__ __forceinline__ int64_t ix_units(const IndexerArgs& a, int32_t q) {
  return ceil_div(clamp_len(a, q), kIxDUnit);
}

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// lane `l`'s value, as a wave-uniform (scalar) value
__device__ __forceinline__ int64_t lane_value(int64_t v, int l) {
  const int64_t x = __shfl(v, l);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <bool kFp8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
indexer_paged_mfma_kernel(IndexerArgs a) {
  constexpr int kRowBytes = kFp8 ? kIxDim : 2 * kIxDim;
  const int lane = threadIdx.x & 63;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kIxWaves + (threadIdx.x >> 6);
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * kIxWaves;

  // ---- this wave's units [u0, u1) and the query holding u0.  Lane l sums
  // the units of queries [l*nb, (l+1)*nb); the lane whose block holds u0
  // is then scanned query by query.
  const int32_t nb = (a.n_q + kWave - 1) / kWave;
  int64_t mine = 0;
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t q = lane * nb + i;
    if (q < a.n_q) mine += ix_units(a, q);
  }
  const int64_t incl = wave_incl_scan(mine, lane);
  const int64_t total = lane_value(incl, kWave - 1);
  const int64_t u0 = g * total / n_waves, u1 = (g + 1) * total / n_waves;
  if (u0 >= u1) return;   // no workgroup barrier in this kernel
  const int l0 = static_cast<int>(__builtin_ctzll(__ballot(incl > u0)));
  int64_t base = lane_value(incl - mine, l0);   // units before query j
  int32_t j = -1;
  for (int32_t c = 0; c < nb && j < 0; c += kWave) {
    const int32_t q = l0 * nb + c + lane;
    const int64_t n = (c + lane < nb && q < a.n_q) ? ix_units(a, q) : 0;
    const int64_t inc = wave_incl_scan(n, lane);
    const uint64_t hit = __ballot(base + inc > u0);
    if (hit != 0ull) {
      const int l = static_cast<int>(__builtin_ctzll(hit));
      j = l0 * nb + c + l;
      base += lane_value(inc - n, l);
    } else {
      base += lane_value(inc, kWave - 1);
    }
  }

  const uint8_t* keys = static_cast<const uint8_t*>(a.k_idx);
  __shared__ __align__(16) uint8_t tiles[kIxWaves][kFp8 ? 16 : 32 * 256];
  uint8_t* tile = tiles[threadIdx.x >> 6];
  for (int64_t u = u0; u < u1 && j < a.n_q; ++j) {
    const int32_t L = clamp_len(a, j);
    const int64_t nj = ceil_div(L, kIxDUnit);
    const int64_t s_begin = u - base;
    const int64_t s_end = nj < u1 - base ? nj : u1 - base;
    base += nj;
    if (s_begin >= s_end) continue;
    u = base - nj + s_end;
    float* srow = a.scores + static_cast<int64_t>(j) * a.score_stride;
    const int32_t req = a.q_req ? a.q_req[j] : 0;
    if (a.k_rows == 0 || req < 0 || req >= a.n_req) {   // every position unmapped
      for (int64_t p = kIxDUnit * s_begin + lane; p < kIxDUnit * s_end && p < L; p += kWave)
        srow[p] = -INFINITY;
      continue;
    }
    const int64_t kv0 = a.kv_start[j];
    const int32_t* table = a.page_table + static_cast<int64_t>(req) * a.max_pages;
    const uint32_t ps = static_cast<uint32_t>(a.page_size);
    // Page lookup of this lane's key in unit s, in two halves: the table
    // load is issued one unit before the row is formed from it, so that the
    // wait for it falls after the MFMAs of the unit in between.  Positions
    // are int32 by interface, so 32-bit division is exact.
    struct PageRef { int32_t pid; uint32_t off; bool ok; };
    auto pt_issue = [&](int64_t s) -> PageRef {
      const int64_t p = kIxDUnit * s + (lane & 31);
      const int64_t l = kv0 + p;
      const uint32_t pg = static_cast<uint32_t>(l) / ps;
      const bool ok = p < L && l >= 0 && pg < static_cast<uint32_t>(a.max_pages);
      return {table[ok ? pg : 0u], static_cast<uint32_t>(l) - pg * ps, ok};
    };
    auto row_from = [&](const PageRef& r) -> int64_t {
      const int64_t row = static_cast<int64_t>(r.pid) * ps + r.off;
      return (r.ok && r.pid >= 0 && row < a.k_rows) ? row : -1;
    };

    const uint16_t* q0 = static_cast<const uint16_t*>(a.q_idx) +
                         static_cast<int64_t>(j) * kIxHeads * kIxDim;
    bf16x8 qa[kIxRowBlocks][kIxKSteps];
#pragma unroll
    for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
      for (int ks = 0; ks < kIxKSteps; ++ks) qa[rb][ks] = load_q_frag(q0, rb, ks, lane);
    // output element i of row block rb in this lane belongs to head
    // 32*rb + 8*(i/4) + 4*(lane/32) + i%4
    float wr[kIxRowBlocks][16];
    const float* wj = a.w + static_cast<int64_t>(j) * kIxHeads;
#pragma unroll
    for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) wr[rb][i] = wj[rb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)];

    // Key loads of one unit.  bf16: instruction i brings 8 whole 128-byte
    // lines, half i%2 of keys (l%8) + 8*(i/2) (lane l takes 16 bytes), so
    // that every request is a full line; the rows are then transposed
    // through this wave's LDS tile into MFMA fragments.  fp8 (128-byte
    // rows): lane l loads its fragment bytes of key l%32 directly.
    // Unmapped keys read row 0 and are masked on write.
    auto issue = [&](int64_t row, u32x4 (&kf)[kIxKSteps]) {
      if constexpr (kFp8) {
        const uint8_t* kp = keys + (row >= 0 ? row : 0) * kRowBytes + (lane >> 5) * 8;
#pragma unroll
        for (int ks = 0; ks < kIxKSteps; ++ks) {
          const uint2 c = *reinterpret_cast<const uint2*>(kp + ks * 16);
          kf[ks] = u32x4{c.x, c.y, 0u, 0u};
        }
      } else {
#pragma unroll
        for (int i = 0; i < kIxKSteps; ++i) {
          const int64_t r = __shfl(row, (lane & 7) + 8 * (i >> 1));
          const uint8_t* kp = keys + (r >= 0 ? r : 0) * kRowBytes + 16 * (lane >> 3) + 128 * (i & 1);
          kf[i] = *reinterpret_cast<const u32x4*>(kp);
        }
      }
    };
    auto step = [&](int64_t s, const u32x4 (&kf)[kIxKSteps], int64_t row) {
      bf16x8 kb[kIxKSteps];
      if constexpr (kFp8) {
#pragma unroll
        for (int ks = 0; ks < kIxKSteps; ++ks) {
          const uint2 lo = fp8x4_to_bf16x4(kf[ks].x);
          const uint2 hi = fp8x4_to_bf16x4(kf[ks].y);
          kb[ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
      } else {
        // tile: key r's 16-byte chunk c at r*256 + 16*(c ^ swz(r)); the
        // swizzle keeps both the line-shaped writes and the fragment reads
        // (16 lanes, 16 keys, one chunk) on distinct banks
        auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };
#pragma unroll
        for (int i = 0; i < kIxKSteps; ++i) {
          const int r = (lane & 7) + 8 * (i >> 1);
          const int c = 8 * (i & 1) + (lane >> 3);
          *reinterpret_cast<u32x4*>(tile + r * 256 + 16 * (c ^ swz(r))) = kf[i];
        }
        const int r = lane & 31;
#pragma unroll
        for (int ks = 0; ks < kIxKSteps; ++ks) {
          const int c = 2 * ks + (lane >> 5);
          kb[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + r * 256 + 16 * (c ^ swz(r))));
        }
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
      float v = 0.f;
#pragma unroll
      for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaf(wr[rb][i], relu_raw(acc[rb][i]), v);
      v += __shfl_xor(v, 32);
      const int64_t p = kIxDUnit * s + lane;
      if (lane < 32 && p < L) {
        if (row < 0) {
          v = -INFINITY;
        } else if constexpr (kFp8) {
          v *= a.k_scale[row >> a.k_scale_shift];
        }
        srow[p] = v;
      }
    };

    // The key loads of unit u+1 are in flight while unit u computes; the
    // table loads run four units ahead of the key loads, so that the row
    // of the next unit is known (its table load long done) when its key
    // loads are issued.  Loads are issued unconditionally (past the last
    // unit they repeat it, from cache) so that every wait is the same in
    // every iteration.
    const int64_t s_last = s_end - 1;
    auto cl = [&](int64_t u) { return u < s_last ? u : s_last; };
    u32x4 k0[kIxKSteps], k1[kIxKSteps];
    int64_t r0 = row_from(pt_issue(s_begin)), r1;
    PageRef pa = pt_issue(cl(s_begin + 1)), pb = pt_issue(cl(s_begin + 2)),
            pc = pt_issue(cl(s_begin + 3)), pd = pt_issue(cl(s_begin + 4));
    issue(r0, k0);
    for (int64_t s = s_begin; s < s_end; s += 4) {
      r1 = row_from(pa);
      pa = pt_issue(cl(s + 5));
      issue(r1, k1);
      step(s, k0, r0);
      if (s + 1 >= s_end) break;
      r0 = row_from(pb);
      pb = pt_issue(cl(s + 6));
      issue(r0, k0);
      step(s + 1, k1, r1);
      if (s + 2 >= s_end) break;
      r1 = row_from(pc);
      pc = pt_issue(cl(s + 7));
      issue(r1, k1);
      step(s + 2, k0, r0);
      if (s + 3 >= s_end) break;
      r0 = row_from(pd);
      pd = pt_issue(cl(s + 8));
      issue(r0, k0);
      step(s + 3, k1, r1);
    }
  }
}

// ------------------------------------------- prefill, balanced persistent path
// The causal work of a prefill is very uneven over (query block, key range)
// pairs: the late query blocks see every key, the early ones a few, and a
// grid of one workgroup per pair leaves about half the workgroups with no
// key at all (each still costs a dispatch and the reads of its ranges) and
// the rest with 1 to 10 tiles.  Here one workgroup per CU takes an equal
// share of the launch's work, in query-block order, and no workgroup is
// empty.  Each step computes one key tile against the 8 queries of the
// current block (8 waves, one query per wave, the tile gathered into LDS by
// DMA, double-buffered).  The walk over tiles:
//   - a query block's tiles are those of its causal key range [lo, hi) (the
//     union of its 8 queries' ranges), cut into windows of kIxBWin keys,
//     each window's tiles starting at its first 64-key half that has work;
//   - the shares are equal in cost, not in tiles: a tile weighs kIxBTileW
//     and entering a block (its query loads, whose latency nothing hides)
//     weighs kIxBBlockW, so a share of many short blocks gets fewer tiles;
//   - scores are staged in LDS per window and written out once the
//     workgroup leaves the window (the next tile is in another window or
//     query block, or its share ends): at the top of the next step, right
//     after its gather, so that the stores complete under its products;
//     fp8 key scales (one per 64-key half, loaded a tile ahead) are applied
//     as the scores are staged;
//   - the gather of the next tile is issued at the top of each step, also
//     when that tile belongs to the next window or query block;
//   - when the query block changes, each wave loads its new query's range
//     during the last tile of the old block, and its A fragments and head
//     weights right after that tile's products.
// Set-up: every workgroup stages the launch's query ranges in LDS
// (coalesced loads, all in flight), computes each query block's range and
// tile count, scans the weights and tile counts, and takes the tiles that
// start in its share [W*b/G, W*(b+1)/G) of the total weight W.
constexpr int32_t kIxBWin = 2048;    // keys per score window
constexpr int kIxBMaxQb = 1024;      // query blocks per launch
constexpr int kIxBPerCu = 1;         // resident workgroups per CU

template <bool kFp8>
__device__ __forceinline__ void ix_window(int32_t lo, int32_t len, int64_t w, int64_t& tfirst,
                                          int32_t& ntiles) {
  constexpr int kTile = IxTile<kFp8>::kTile;
  const int64_t hi = static_cast<int64_t>(lo) + len;
  const int64_t wlo = w * kIxBWin > lo ? w * kIxBWin : lo;
  const int64_t whi = (w + 1) * kIxBWin < hi ? (w + 1) * kIxBWin : hi;
  tfirst = (wlo / kIxPHalf) * kIxPHalf;
  ntiles = static_cast<int32_t>(ceil_div(whi - tfirst, kTile));
}

// tiles of a block with union range [lo, lo + len): the sum of ix_window's
// counts over the windows the range touches
template <bool kFp8>
__device__ __forceinline__ int64_t ix_block_tiles(int32_t lo, int32_t len) {
  constexpr int kTile = IxTile<kFp8>::kTile;
  if (len <= 0) return 0;
  const int64_t hi = static_cast<int64_t>(lo) + len;
  const int64_t w0 = lo / kIxBWin, w1 = (hi - 1) / kIxBWin;
  const int64_t t0 = (lo / kIxPHalf) * kIxPHalf;
  if (w0 == w1) return ceil_div(hi - t0, kTile);
  return ceil_div((w0 + 1) * kIxBWin - t0, kTile) + (w1 - w0 - 1) * (kIxBWin / kTile) +
         ceil_div(hi - w1 * kIxBWin, kTile);
}

// causal key range [lo, hi) of query j, clamped to the key rows (hi <= lo:
// no work)
__device__ __forceinline__ void ix_query_range(const IndexerArgs& a, int32_t j, int64_t& lo,
                                               int64_t& hi) {
  lo = 0;
  hi = 0;
  if (j < a.n_q) {
    lo = a.kv_start[j];
    hi = lo + clamp_len(a, j);
    if (lo < 0) lo = 0;
    if (hi > a.k_rows) hi = a.k_rows;
    if (hi < lo) hi = lo;
  }
}

template <bool kFp8>
__global__ void __launch_bounds__(kWave * kIxPWaves)
indexer_prefill_balanced_kernel(IndexerArgs a, int32_t qb0, int32_t n_qb) {
  using TL = IxTile<kFp8>;
  constexpr int kTile = TL::kTile;
  constexpr int kHalves = kTile / kIxPHalf;
  // a 64-key half's products take about 3.3K clocks on the two waves of a
  // SIMD; a block entry exposes one memory latency (about 7K clocks)
  constexpr int64_t kIxBTileW = kFp8 ? 2 : 1;
  constexpr int64_t kIxBBlockW = 1;
  static_assert(kIxBWin % kTile == 0 && kIxBWin % kFp8BlockRows == 0,
                "windows hold whole tiles and whole fp8 scale blocks");
  static_assert(kIxPHalf <= kFp8BlockRows && kFp8BlockRows % kIxPHalf == 0,
                "a 64-key half has one fp8 scale");
  __shared__ float sc[kIxPWaves][kIxBWin];                  // scores of the current window
  __shared__ int32_t qb_lo[kIxBMaxQb], qb_len[kIxBMaxQb];   // union range of each block
  __shared__ int64_t wave_tot[2][kIxPWaves];
  __shared__ int64_t share_tiles[2];                        // tiles starting before g0, g1
  __shared__ int32_t first_qb, first_off;
  __shared__ int64_t first_lo[kIxPWaves], first_hi[kIxPWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- set-up: ranges, tiles and weights of this thread's kBPT blocks
  // (kBPT*tid ...).  The launch's query ranges are staged in LDS first (in
  // the tile buffers, free until the walk) with coalesced loads, all in
  // flight.
  constexpr int kBPT = kIxBMaxQb / (kWave * kIxPWaves);   // query blocks per thread
  constexpr int kQPT = kBPT * kIxPWaves;                    // their queries
  static_assert(kBPT * kWave * kIxPWaves == kIxBMaxQb, "whole blocks per thread");
  static_assert(sizeof(int32_t) * kIxBMaxQb * kIxPWaves <= kIxBufBytes, "the ranges fit a tile buffer");
  int64_t ql[kQPT], qh[kQPT];
  {
    int32_t* s_start = reinterpret_cast<int32_t*>(g_ix_buf0);
    int32_t* s_len = reinterpret_cast<int32_t*>(g_ix_buf1);
    const int32_t j0 = qb0 * kIxPWaves;
    const int32_t nj = a.n_q - j0 < n_qb * kIxPWaves ? a.n_q - j0 : n_qb * kIxPWaves;
    int32_t vs[kQPT], vl[kQPT];
#pragma unroll
    for (int u = 0; u < kQPT; ++u) {
      const int32_t i = u * kWave * kIxPWaves + tid;
      const int32_t ic = i < nj ? i : nj - 1;
      vs[u] = a.kv_start[j0 + ic];
      vl[u] = a.kv_len[j0 + ic];
    }
#pragma unroll
    for (int u = 0; u < kQPT; ++u) {
      const int32_t i = u * kWave * kIxPWaves + tid;
      if (i < nj) {
        s_start[i] = vs[u];
        s_len[i] = vl[u];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQPT; ++i) {
      const int32_t q = kBPT * tid + i / kIxPWaves;
      const int32_t jl = q * kIxPWaves + i % kIxPWaves;
      const bool in = q < n_qb && jl < nj;
      const int32_t st = in ? s_start[jl] : 0, ln = in ? s_len[jl] : 0;
      const int64_t lo = st < 0 ? 0 : st;
      int64_t hi = static_cast<int64_t>(st) + (ln < 0 ? 0 : (ln > a.max_kv_len ? a.max_kv_len : ln));
      hi = hi > a.k_rows ? a.k_rows : hi;
      const bool ok = in && hi > lo;
      ql[i] = ok ? lo : 0;
      qh[i] = ok ? hi : 0;
    }
  }
  int64_t nt[kBPT], wt[kBPT], sum_w = 0, sum_t = 0;
#pragma unroll
  for (int k = 0; k < kBPT; ++k) {
    int64_t lo = INT64_MAX, hi = 0;
#pragma unroll
    for (int i = kIxPWaves * k; i < kIxPWaves * (k + 1); ++i) {
      if (qh[i] > ql[i]) {
        lo = ql[i] < lo ? ql[i] : lo;
        hi = qh[i] > hi ? qh[i] : hi;
      }
    }
    const int32_t len = hi > lo ? static_cast<int32_t>(hi - lo) : 0;
    const int32_t l32 = hi > lo ? static_cast<int32_t>(lo) : 0;
    nt[k] = ix_block_tiles<kFp8>(l32, len);
    wt[k] = nt[k] > 0 ? kIxBTileW * nt[k] + kIxBBlockW : 0;
    sum_w += wt[k];
    sum_t += nt[k];
    const int32_t q = kBPT * tid + k;
    if (q < n_qb) {
      qb_lo[q] = l32;
      qb_len[q] = len;
    }
  }
  const int64_t incl_w = wave_incl_scan(sum_w, lane);
  const int64_t incl_t = wave_incl_scan(sum_t, lane);
  if (lane == kWave - 1) {
    wave_tot[0][wave] = incl_w;
    wave_tot[1][wave] = incl_t;
  }
  __syncthreads();
  int64_t bw = 0, bt = 0, sw = 0, stt = 0;
#pragma unroll
  for (int w = 0; w < kIxPWaves; ++w) {
    const int64_t x = wave_tot[0][w], y = wave_tot[1][w];
    bw += w < wave ? x : 0;
    bt += w < wave ? y : 0;
    sw += x;
    stt += y;
  }
  const int64_t w_total = lane_value(sw, 0), t_total = lane_value(stt, 0);
  if (w_total == 0) return;
  // weight and tile prefixes of this thread's blocks
  int64_t pw[kBPT], pt[kBPT];
  pw[0] = bw + incl_w - sum_w;
  pt[0] = bt + incl_t - sum_t;
#pragma unroll
  for (int k = 1; k < kBPT; ++k) {
    pw[k] = pw[k - 1] + wt[k - 1];
    pt[k] = pt[k - 1] + nt[k - 1];
  }
  const int64_t g0 = w_total * blockIdx.x / gridDim.x;
  const int64_t g1 = w_total * (blockIdx.x + 1) / gridDim.x;
  // tile i of a block starts at weight pw + kIxBBlockW + i * kIxBTileW and
  // belongs to the share its start falls in: count the tiles starting
  // before g0 and before g1
#pragma unroll
  for (int k = 0; k < kBPT; ++k) {
    auto before = [&](int64_t g) {
      int64_t c = g - pw[k] - kIxBBlockW;
      c = c <= 0 ? 0 : ceil_div(c, kIxBTileW);
      return pt[k] + (c < nt[k] ? c : nt[k]);
    };
    if (wt[k] > 0 && pw[k] <= g0 && g0 < pw[k] + wt[k]) share_tiles[0] = before(g0);
    if (wt[k] > 0 && pw[k] <= g1 && g1 < pw[k] + wt[k]) share_tiles[1] = before(g1);
  }
  if (tid == 0 && g1 >= w_total) share_tiles[1] = t_total;
  __syncthreads();
  const int64_t f0 = lane_value(share_tiles[0], 0), f1 = lane_value(share_tiles[1], 0);
  if (f1 <= f0) return;   // the whole workgroup: no barrier below is skipped by part of it
  // the block holding tile f0 (the share's first), and its queries' ranges
#pragma unroll
  for (int k = 0; k < kBPT; ++k) {
    if (nt[k] > 0 && pt[k] <= f0 && f0 < pt[k] + nt[k]) {
      first_qb = kBPT * tid + k;
      first_off = static_cast<int32_t>(f0 - pt[k]);
#pragma unroll
      for (int i = 0; i < kIxPWaves; ++i) {
        first_lo[i] = ql[kIxPWaves * k + i];
        first_hi[i] = qh[kIxPWaves * k + i];
      }
    }
  }
  __syncthreads();

  // ---- walk state (wave-uniform): block qb, window w, tile t of the
  // window's n_t tiles starting at row tf
  struct Pos {
    int32_t qb, t, n_t;
    int64_t w, tf;
  };
  auto block_lo = [&](int32_t q) { return __builtin_amdgcn_readfirstlane(qb_lo[q]); };
  auto block_len = [&](int32_t q) { return __builtin_amdgcn_readfirstlane(qb_len[q]); };
  auto enter_window = [&](Pos& p) { ix_window<kFp8>(block_lo(p.qb), block_len(p.qb), p.w, p.tf, p.n_t); };
  auto advance = [&](Pos p) {
    if (p.t + 1 < p.n_t) {
      ++p.t;
      return p;
    }
    p.t = 0;
    const int32_t lo = block_lo(p.qb), len = block_len(p.qb);
    if ((p.w + 1) * kIxBWin < static_cast<int64_t>(lo) + len) {
      ++p.w;
    } else {
      // next block with work (there is one: the share has tiles left; the
      // bound keeps the walk inside the launch's blocks regardless)
      do {
        ++p.qb;
      } while (p.qb + 1 < n_qb && block_len(p.qb) == 0);
      p.w = block_lo(p.qb) / kIxBWin;
    }
    enter_window(p);
    return p;
  };
  Pos cur;
  cur.qb = __builtin_amdgcn_readfirstlane(first_qb);
  cur.w = block_lo(cur.qb) / kIxBWin;
  cur.t = 0;
  enter_window(cur);
  {
    int32_t off = __builtin_amdgcn_readfirstlane(first_off);
    // (every window of a block with work has at least one tile; the second
    // condition only bounds the loop)
    while (off >= cur.n_t && cur.n_t > 0) {
      off -= cur.n_t;
      ++cur.w;
      enter_window(cur);
    }
    cur.t = off;
  }

  // this wave's query in the current block: range, A fragments, weights
  auto query_of = [&](int32_t q) { return (qb0 + q) * kIxPWaves + wave; };
  int64_t my_lo = lane_value(first_lo[wave], 0), my_hi = lane_value(first_hi[wave], 0);
  bf16x8 qa[kIxRowBlocks][kIxKSteps];
  float wv[kIxRowBlocks][16];
  auto load_query = [&](int32_t j, bool live) {
    const uint16_t* q0 = static_cast<const uint16_t*>(a.q_idx) +
                         static_cast<int64_t>(live ? j : 0) * kIxHeads * kIxDim;
    const float* w0 = a.w + static_cast<int64_t>(live ? j : 0) * kIxHeads;
#pragma unroll
    for (int rb = 0; rb < kIxRowBlocks; ++rb) {
#pragma unroll
      for (int ks = 0; ks < kIxKSteps; ++ks) qa[rb][ks] = load_q_frag(q0, rb, ks, lane);
#pragma unroll
      for (int i = 0; i < 16; ++i) wv[rb][i] = w0[rb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)];
    }
  };
  // fp8 key scales of a tile's 64-key halves, loaded one tile ahead (the
  // top-of-step wait covers them); a tile's buffer parity picks the set
  float ksc[2][kHalves];
  auto load_scales = [&](float (&dst)[kHalves], int64_t base) {
    if constexpr (kFp8) {
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        int64_t r = base + hf * kIxPHalf;
        r = r < a.k_rows ? r : a.k_rows - 1;
        dst[hf] = a.k_scale[r / kFp8BlockRows];
      }
    }
  };
  const uint8_t* keys = static_cast<const uint8_t*>(a.k_idx);
  IxSlots<kFp8> sl;
  sl.init(wave, lane);
  // the first tile's gather goes out with the query loads (the first
  // step's wait covers both)
  load_query(query_of(cur.qb), my_hi > my_lo);
  load_scales(ksc[0], cur.tf + static_cast<int64_t>(cur.t) * kTile);
  ix_issue_tile<0, kFp8>(keys, a.k_rows, cur.tf + static_cast<int64_t>(cur.t) * kTile, sl, wave);

  int64_t left = f1 - f0;        // tiles of the share not yet computed
  int32_t seg_t0 = cur.t;        // first tile of the current window computed here
  // This wave's scores of rows [lo, hi) of the window starting at row c_lo
  // go to its query's score row (position = row - q_lo), all LDS reads of a
  // group of four rows per lane ahead of its stores.
  auto flush = [&](int64_t lo, int64_t hi, int64_t c_lo, float* srow, int64_t q_lo) {
    for (int64_t r0 = lo; r0 < hi; r0 += 4 * kWave) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t r = r0 + u * kWave + lane;
        v[u] = r < hi ? sc[wave][r - c_lo] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t r = r0 + u * kWave + lane;
        if (r < hi) srow[r - q_lo] = v[u];
      }
    }
  };
  // A window's flush waits for the next step (when the workgroup has one):
  // issued there right after the next gather, the stores then complete
  // under that step's products instead of delaying its top-of-step wait.
  int64_t fl_lo = 0, fl_hi = 0, fl_clo = 0, fl_qlo = 0;
  float* fl_row = a.scores;
  auto step = [&](auto bufc) {
    constexpr int B = decltype(bufc)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's gather of this tile landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();         // every wave's; the other buffer fully consumed
    asm volatile("" ::: "memory");
    const bool more = left > 1;
    Pos nxt = cur;
    if (more) {
      nxt = advance(cur);
      const int64_t nbase = nxt.tf + static_cast<int64_t>(nxt.t) * kTile;
      ix_issue_tile<1 - B, kFp8>(keys, a.k_rows, nbase, sl, wave);
      load_scales(ksc[1 - B], nbase);
    }
    if (fl_hi > fl_lo) {   // the previous window's rows (read before this step's score writes)
      flush(fl_lo, fl_hi, fl_clo, fl_row, fl_qlo);
      fl_hi = fl_lo;
    }
    const bool new_block = more && nxt.qb != cur.qb;
    int64_t nx_lo = my_lo, nx_hi = my_hi;
    if (new_block) ix_query_range(a, query_of(nxt.qb), nx_lo, nx_hi);

    const bool live = my_hi > my_lo;
    const int64_t c_lo = cur.w * kIxBWin, c_hi = c_lo + kIxBWin;
    const int64_t base = cur.tf + static_cast<int64_t>(cur.t) * kTile;
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      const int64_t hbase = base + hf * kIxPHalf;
      // (a window's last tile can reach past the window: those rows are
      // the next window's)
      if (!live || hbase >= my_hi || hbase + kIxPHalf <= my_lo || hbase >= c_hi) continue;
      const uint8_t* tile = ix_buf<B>() + hf * kIxPHalf * TL::kLdsRow;
      f32x16 acc[2][kIxRowBlocks];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][rb][i] = 0.f;
      // The two waves of a SIMD leave each barrier together and would run
      // their products and their head sums in step; a raised priority for
      // the products lets a wave in its head sum yield the issue slots to
      // the other's MFMAs, so the vector work fills the matrix core's gaps.
      __builtin_amdgcn_s_setprio(1);
      bf16x8 b0 = ix_bfrag<kFp8>(tile, 0, 0, lane), b1 = ix_bfrag<kFp8>(tile, 1, 0, lane);
#pragma unroll
      for (int ks = 0; ks < kIxKSteps; ++ks) {
        bf16x8 n0 = b0, n1 = b1;
        if (ks + 1 < kIxKSteps) {
          n0 = ix_bfrag<kFp8>(tile, 0, ks + 1, lane);
          n1 = ix_bfrag<kFp8>(tile, 1, ks + 1, lane);
        }
#pragma unroll
        for (int rb = 0; rb < kIxRowBlocks; ++rb) {
          acc[0][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][ks], b0, acc[0][rb], 0, 0, 0);
          acc[1][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[rb][ks], b1, acc[1][rb], 0, 0, 0);
        }
        b0 = n0;
        b1 = n1;
        if constexpr (!kFp8) __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float v = 0.f;
#pragma unroll
        for (int rb = 0; rb < kIxRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) v = fmaf(wv[rb][i], relu_raw(acc[nb][rb][i]), v);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                         false, false);
        v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if constexpr (kFp8) v *= ksc[B][hf];   // the key rows' fp8 scale
        const int64_t row = hbase + nb * 32 + (lane & 31);
        if (lane < 32 && row >= my_lo && row < my_hi && row < c_hi) sc[wave][row - c_lo] = v;
      }
    }
    // leaving the window: this wave's scores of the rows computed here
    // (tiles seg_t0..t of the window) go out, at the next step's top or,
    // at the end of the share, now
    if (!more || nxt.qb != cur.qb || nxt.w != cur.w) {
      if (live) {
        int64_t lo = cur.tf + static_cast<int64_t>(seg_t0) * kTile;
        int64_t hi = base + kTile;
        lo = lo > my_lo ? lo : my_lo;
        hi = hi < my_hi ? hi : my_hi;
        hi = hi < c_hi ? hi : c_hi;
        float* srow = a.scores + static_cast<int64_t>(query_of(cur.qb)) * a.score_stride;
        if (more) {
          fl_lo = lo;
          fl_hi = hi;
          fl_clo = c_lo;
          fl_row = srow;
          fl_qlo = my_lo;
        } else {
          flush(lo, hi, c_lo, srow, my_lo);
        }
      }
      seg_t0 = nxt.t;
    }
    if (new_block) {
      my_lo = nx_lo;
      my_hi = nx_hi;
      load_query(query_of(nxt.qb), my_hi > my_lo);
    }
    cur = nxt;
    --left;
  };
  while (true) {
    step(std::integral_constant<int, 0>{});
    if (left == 0) break;
    step(std::integral_constant<int, 1>{});
    if (left == 0) break;
  }
}

// ------------------------------------------------------------------ host


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
    // about two resident workgroups per CU, at least a few units per wave
    const int64_t units_max = static_cast<int64_t>(a.n_q) * ceil_div(a.max_kv_len, kIxDUnit);
    int64_t blocks = 2 * static_cast<int64_t>(device_cu_count());
    const int64_t by_work = ceil_div(units_max, 4 * kIxWaves);
    blocks = by_work < blocks ? by_work : blocks;
    if (fp8) indexer_paged_mfma_kernel<true><<<blocks, kWave * kIxWaves, 0, s>>>(a);
    else indexer_paged_mfma_kernel<false><<<blocks, kWave * kIxWaves, 0, s>>>(a);
    return check_launch("indexer_scores (paged)");
  }
  // one workgroup per CU, each an equal share of the key tiles of up to
  // kIxBMaxQb query blocks per launch
  const int32_t n_qblocks = static_cast<int32_t>(ceil_div(a.n_q, kIxPWaves));
  const unsigned grid = static_cast<unsigned>(device_cu_count() * kIxBPerCu);
  for (int32_t qb0 = 0; qb0 < n_qblocks; qb0 += kIxBMaxQb) {
    const int32_t n = n_qblocks - qb0 < kIxBMaxQb ? n_qblocks - qb0 : kIxBMaxQb;
    if (fp8)
      indexer_prefill_balanced_kernel<true><<<grid, kWave * kIxPWaves, 0, s>>>(a, qb0, n);
    else
      indexer_prefill_balanced_kernel<false><<<grid, kWave * kIxPWaves, 0, s>>>(a, qb0, n);
    const ds_status st = check_launch("indexer_scores (prefill)");
    if (st != DS_OK) return st;
  }
  return DS_OK;
}

}  // namespace ds32cp
