// Step 5: sparse latent attention (MLA) over each query's selected rows.
//
// Sources: "[RFC]: Parallel strategy for Deepseek v3.2 like models" --
// comment thread (each query attends only to its top-k KV entries instead
// of all KV), "Pros" (all heads stay on one rank, so the attention is a
// dense, high-intensity contraction); "Model Parallel Strategy Analysis",
// common-errors table (MLA's compressed KV is one latent vector per
// token, shared by every head).  Reading (the pages give no formula):
// absorbed latent form, key = the full latent row (d_latent + d_rope),
// value = its first d_latent columns,
//   out[j,h,:] = sum_s softmax_s(sm_scale * <q[j,h,:], kv[s,:]>) kv[s,:d_latent]
//   lse[j,h]   = log sum_s exp(sm_scale * <q[j,h,:], kv[s,:]>).
//
// Kernels (d_latent 512, d_rope 64; 32, 64 or 128 heads):
//   * mla_bf16_wide_kernel: bf16 rows (and fp8 prefill rows, widened once
//     per call into the workspace).  One workgroup per (query, split of its
//     selected rows), one wave per 32 heads and per SIMD; 32-row tiles of
//     the selected rows are gathered into LDS by DMA and serve all heads as
//     key (QK) and value (PV) on v_mfma_f32_16x16x32_bf16.
//   * mla_fp8_kernel: fp8 rows read in place (decode pools), widened to
//     bf16 exactly in LDS; the row scales are applied in fp32.
//   * mla_f32_kernel: the all-fp32 path of the tiny workload.
// Decode (few queries) splits each query's selected rows over several
// workgroups that write unnormalised partial outputs with their running
// max and sum; mla_combine_kernel merges them by log-sum-exp.
#include <type_traits>
#include <utility>

#include "common.h"

namespace ds32cp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ fp32
// One workgroup per (query, head): logits of every selected row in LDS,
// then a block softmax and one output column per thread.
__global__ void __launch_bounds__(256)
mla_f32_kernel(MlaArgs a) {
  extern __shared__ float smem[];
  const int D = a.d_latent + a.d_rope;
  float* qh = smem;               // [D]
  float* logit = smem + D;        // [topk]
  int32_t* rows = reinterpret_cast<int32_t*>(logit + a.topk);   // [topk]
  __shared__ float red[256 / kWave];
  __shared__ float sh_max, sh_sum;

  const int32_t j = blockIdx.x;
  const int32_t h = blockIdx.y;
  const int tid = threadIdx.x;
  const float* q = static_cast<const float*>(a.q) +
                   (static_cast<int64_t>(j) * a.n_heads + h) * D;
  const float* kv = static_cast<const float*>(a.kv);
  for (int i = tid; i < D; i += blockDim.x) qh[i] = q[i];
  __syncthreads();
  float mx = -INFINITY;
  for (int s = tid; s < a.topk; s += blockDim.x) {
    int32_t r = a.topk_idx[static_cast<int64_t>(j) * a.topk + s];
    if (r >= a.kv_rows) r = -1;
    rows[s] = r;
    float l = -INFINITY;
    if (r >= 0) {
      const float* k = kv + static_cast<int64_t>(r) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qh[d], k[d], dot);
      l = dot * a.sm_scale;
    }
    logit[s] = l;
    mx = fmaxf(mx, l);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
    for (int w = 1; w < static_cast<int>(blockDim.x / kWave); ++w) m = fmaxf(m, red[w]);
    sh_max = m;
  }
  __syncthreads();
  const float m = sh_max;
  float sum = 0.f;
  for (int s = tid; s < a.topk; s += blockDim.x) {
    const float p = rows[s] >= 0 ? expf(logit[s] - m) : 0.f;
    logit[s] = p;
    sum += p;
  }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < static_cast<int>(blockDim.x / kWave); ++w) t += red[w];
    sh_sum = t;
  }
  __syncthreads();
  const float total = sh_sum;
  const float inv = total > 0.f ? 1.f / total : 0.f;
  float* out = static_cast<float*>(a.out) + (static_cast<int64_t>(j) * a.n_heads + h) * a.d_latent;
  for (int c = tid; c < a.d_latent; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < a.topk; ++s) {
      if (rows[s] < 0) continue;
      acc = fmaf(logit[s], kv[static_cast<int64_t>(rows[s]) * D + c], acc);
    }
    out[c] = acc * inv;
  }
  if (a.lse && tid == 0)
    a.lse[static_cast<int64_t>(j) * a.n_heads + h] = total > 0.f ? m + logf(total) : -INFINITY;
}

// --------------------------------------------------------- MFMA constants
constexpr int kMlaDl = 512;
constexpr int kMlaDr = 64;
constexpr int kMlaD = kMlaDl + kMlaDr;            // 576
constexpr int kMlaKSteps = kMlaD / 32;            // 18 QK steps of K = 32
constexpr int kMlaCBlocks = kMlaDl / 16;          // 32 output column blocks
constexpr int kMlaTile = 64;                      // selected rows per tile
constexpr int kMlaRowBytes = kMlaD * 2;           // 1152 (bf16 row)
constexpr int kMlaRowChunks = kMlaRowBytes / 16;  // 72
constexpr int kMlaLdsRow = kMlaRowBytes + 16;     // padded LDS row stride

// ---- split partials (decode): O unnormalised in bf16 [n_q, n_splits, H,
// Dl], then (m, l) in fp32 [n_q, n_splits, H, 2] from a 256-byte boundary
__host__ __device__ inline size_t mla_partial_o_bytes(int64_t n_q, int64_t n_splits,
                                                      int64_t n_heads) {
  return static_cast<size_t>(round_up(n_q * n_splits * n_heads * kMlaDl * 2, 256));
}
__device__ __forceinline__ uint16_t* mla_partial_o(const MlaArgs& a, int32_t j, int32_t split,
                                                   int32_t h) {
  return static_cast<uint16_t*>(a.ws) +
         ((static_cast<int64_t>(j) * a.n_splits + split) * a.n_heads + h) * kMlaDl;
}
__device__ __forceinline__ float* mla_partial_ml(const MlaArgs& a, int32_t j, int32_t split,
                                                 int32_t h) {
  return reinterpret_cast<float*>(static_cast<uint8_t*>(a.ws) +
                                  mla_partial_o_bytes(a.n_q, a.n_splits, a.n_heads)) +
         ((static_cast<int64_t>(j) * a.n_splits + split) * a.n_heads + h) * 2;
}
// four consecutive fp32 outputs -> four bf16 (round to nearest even)
__device__ __forceinline__ void mla_store_bf16x4(uint16_t* p, float x0, float x1, float x2, float x3) {
  uint2 pk;
  pk.x = f32_to_bf16_bits(x0) | (static_cast<uint32_t>(f32_to_bf16_bits(x1)) << 16);
  pk.y = f32_to_bf16_bits(x2) | (static_cast<uint32_t>(f32_to_bf16_bits(x3)) << 16);
  *reinterpret_cast<uint2*>(p) = pk;
}

// Byte offset of 16-byte chunk `c` of tile row `r`.  The 16-byte pad makes
// consecutive rows start 36 banks apart, so 16 lanes reading one chunk of
// 16 consecutive rows (K fragments) and 16 lanes reading 4 rows x 32 bytes
// (transposed V fragments) both hit distinct banks, and every fragment
// address is a per-lane base plus a compile-time offset.
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * kMlaLdsRow + (c << 4);
}

// ------------------------------------------------------ fp8 KV (decode)
// One workgroup of n_heads/16 waves per (query, split of its rows); wave w
// owns heads 16w .. 16w+15.  The split's rows are gathered 64 at a time
// into LDS and widened to bf16 exactly (unit scale: every e4m3fn code is a
// bf16 value); the per-block scale of a row multiplies its logits (before
// the softmax) and its softmax weight (before PV), both in fp32, so the
// arithmetic is on the codes exactly as stored.
//   S^T[key, head] = K[key, :] . Q[head, :]     A = K (LDS), B = Q (regs)
//   O^T[c, head]  += V^T[c, key] . P^T[key, head]
// The transposed form makes the QK output layout (one head per lane, four
// keys per lane) exactly the B operand layout PV needs, so P never leaves
// registers; O^T (16 heads x 512) is 128 accumulator registers per lane and
// each lane owns one head, so a rescale is one scalar per lane.
//
// Lazy rescaling: the running reference max of a head only moves when a
// tile's max exceeds it by more than 2^kRescaleLog2, so that exp2 of any
// logit minus the reference stays below 2^8 and the output accumulator is
// rescaled only on the rare tiles that raise the max.
constexpr float kRescaleLog2 = 8.f;

__global__ void __launch_bounds__(kWave * 8)
mla_fp8_kernel(MlaArgs a, int32_t keys_per_split) {
  __shared__ __align__(16) uint8_t tile[kMlaTile * kMlaLdsRow];
  __shared__ int32_t rows[kMlaTile];
  __shared__ float kscale[kMlaTile];
  __shared__ int32_t any_valid;

  const int32_t j = blockIdx.x / a.n_splits;
  const int32_t split = blockIdx.x - j * a.n_splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int grp = lane >> 4;                      // 0..3
  const int h = wave * 16 + (lane & 15);          // this lane's head

  const int32_t s_begin = split * keys_per_split;
  int32_t s_end = s_begin + keys_per_split;
  s_end = s_end < a.topk ? s_end : a.topk;

  // Q^T fragments (B operand): head h, dims 32*ks + 8*grp + 0..7.
  bf16x8 qf[kMlaKSteps];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<int64_t>(j) * a.n_heads + h) * kMlaD + grp * 8;
#pragma unroll
    for (int ks = 0; ks < kMlaKSteps; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + ks * 32));
  }

  f32x4 o[kMlaCBlocks];
  float m_ref = -INFINITY;   // reference max (log2 domain)
  float l_run = 0.f;         // sum of exp2(logit - m_ref)
#pragma unroll
  for (int cb = 0; cb < kMlaCBlocks; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t* kv = static_cast<const uint8_t*>(a.kv);

  for (int32_t t0 = s_begin; t0 < s_end; t0 += kMlaTile) {
    // ---- gather the tile's rows into LDS
    if (tid < kMlaTile) {
      const int32_t s = t0 + tid;
      int32_t r = s < s_end ? a.topk_idx[static_cast<int64_t>(j) * a.topk + s] : -1;
      if (r >= a.kv_rows) r = -1;
      rows[tid] = r;
      kscale[tid] = r >= 0 ? a.kv_scale[r >> a.scale_shift] : 1.f;
      const uint64_t b = __ballot(r >= 0);
      if (tid == 0) any_valid = b != 0ull;
    }
    __syncthreads();
    if (!any_valid) {
      __syncthreads();
      continue;
    }
    constexpr int kPieces = kMlaTile * (kMlaD / 16);   // 16 codes per piece
    for (int piece = tid; piece < kPieces; piece += nthreads) {
      const int r = piece / (kMlaD / 16);
      const int c8 = piece - r * (kMlaD / 16);
      const int32_t row = rows[r];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row >= 0)
        v = *reinterpret_cast<const uint4*>(kv + static_cast<int64_t>(row) * kMlaD + c8 * 16);
      const uint2 a0 = fp8x4_to_bf16x4(v.x), a1 = fp8x4_to_bf16x4(v.y);
      const uint2 a2 = fp8x4_to_bf16x4(v.z), a3 = fp8x4_to_bf16x4(v.w);
      *reinterpret_cast<uint4*>(&tile[tile_off(r, 2 * c8)]) = make_uint4(a0.x, a0.y, a1.x, a1.y);
      *reinterpret_cast<uint4*>(&tile[tile_off(r, 2 * c8 + 1)]) = make_uint4(a2.x, a2.y, a3.x, a3.y);
    }
    __syncthreads();

    // ---- S^T = K Q^T for 4 blocks of 16 keys
    f32x4 st[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = kb * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < kMlaKSteps; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&tile[tile_off(r, ks * 4 + grp)]));
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], st[kb], 0, 0, 0);
      }
    }

    // ---- online softmax; this lane: head h, keys 16*kb + 4*grp + i
    bf16x8 pb[2];
    {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb * 16 + grp * 4 + i;
          float l = st[kb][i] * scale2 * kscale[key];
          l = rows[key] >= 0 ? l : -INFINITY;
          st[kb][i] = l;
          mx = fmaxf(mx, l);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // move the reference only when needed (uniform over the wave)
      const bool need = mx > m_ref + kRescaleLog2;
      if (__ballot(need)) {
        const float m_new = need ? mx : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 when m_ref = -inf
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < kMlaCBlocks; ++cb) o[cb] *= alpha;
        m_ref = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = __builtin_amdgcn_exp2f(st[kb][i] - m_ref);
          psum += p;
          p *= kscale[kb * 16 + grp * 4 + i];   // fold the row scale into P
          pb[kb >> 1][(kb & 1) * 4 + i] = static_cast<__bf16>(p);
        }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run += psum;
    }

    // ---- O^T += V^T P^T, two steps of 32 keys
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int r0 = (2 * kp) * 16 + grp * 4;       // keys r0..r0+3
      const int r1 = (2 * kp + 1) * 16 + grp * 4;   // keys r1..r1+3
#pragma unroll
      for (int cb = 0; cb < kMlaCBlocks; ++cb) {
        // ds_read_b64_tr_b16: in each 16-lane group, lane i names 4
        // consecutive bf16 of row (base + i/4), columns 4*(i%4)..+3 of the
        // 16-column block; lane i receives column i of the 4 rows.
        const int li = lane & 15;
        const int chunk = 2 * cb + ((li & 3) >> 1);
        const int sub = (li & 1) * 8;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(&tile[tile_off(r0 + (li >> 2), chunk) + sub]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(&tile[tile_off(r1 + (li >> 2), chunk) + sub]));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[kp], o[cb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue
  if (a.n_splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t obase = (static_cast<int64_t>(j) * a.n_heads + h) * kMlaDl + grp * 4;
    if (a.out_dtype == DS_BF16) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
      for (int cb = 0; cb < kMlaCBlocks; ++cb)
        mla_store_bf16x4(out + cb * 16, o[cb][0] * inv, o[cb][1] * inv, o[cb][2] * inv, o[cb][3] * inv);
    } else {
      float* out = static_cast<float*>(a.out) + obase;
#pragma unroll
      for (int cb = 0; cb < kMlaCBlocks; ++cb)
        *reinterpret_cast<float4*>(out + cb * 16) =
            make_float4(o[cb][0] * inv, o[cb][1] * inv, o[cb][2] * inv, o[cb][3] * inv);
    }
    if (a.lse && grp == 0)
      a.lse[static_cast<int64_t>(j) * a.n_heads + h] =
          l_run > 0.f ? (m_ref + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    uint16_t* po = mla_partial_o(a, j, split, h) + grp * 4;
#pragma unroll
    for (int cb = 0; cb < kMlaCBlocks; ++cb)
      mla_store_bf16x4(po + cb * 16, o[cb][0], o[cb][1], o[cb][2], o[cb][3]);
    if (grp == 0) {
      float* pml = mla_partial_ml(a, j, split, h);
      pml[0] = m_ref;
      pml[1] = l_run;
    }
  }
}

// ------------------------------------------- tiles of the bf16 kernel
constexpr int kPipeTile = 32;                                     // rows per tile
constexpr int kMlaMaxKeys = 2048;

// Three tile buffers.  The gathers into them are issued as instructions the
// compiler does not see (wide_gather_issue), so it inserts no wait for them
// before reading a buffer; the kernel waits for its gathers itself (vmcnt
// before the barrier that opens a tile).  A buffer holds one 36 KB tile;
// the stride leaves 1 KB between buffers.
constexpr int kPipeTileBytes = kPipeTile * (kMlaRowBytes + 32);   // 37888
__shared__ __align__(16) uint8_t g_mla_bufs[3 * kPipeTileBytes];

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

// Cross-lane reductions over the four 16-lane rows of a wave (lanes l,
// l^16, l^32, l^48) with the row-swap permutes: no LDS round trip.
__device__ __forceinline__ float mla_rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float mla_rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maxima as the bare instructions: the inputs are finite or -inf, and the
// library's fmaxf would first quiet possible signalling NaNs (one more
// instruction per operand that is not known to be canonical).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order:
// a loop whose index is a constant expression in the body.
template <class F, int... U>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------- bf16 KV, 32 heads per wave
// One workgroup of kNW = n_heads/32 waves (one per SIMD) per (query, split
// of its rows).  Wave w computes S^T for 32 heads (two 16-head MFMA blocks
// share every K fragment read from LDS, so the LDS read traffic of QK is
// half that of 16 heads per wave, the bound of that form), and PV for
// output columns [w*512/kNW, (w+1)*512/kNW) of every head: O^T is (512/kNW)
// x 32kNW / 64 lanes = 256 fp32 per lane, held in the accumulator
// registers (one wave per SIMD has 512), next to the 128 VGPRs of Q^T.
//
// Softmax reference: the logits of a head are taken relative to its
// maximum over the first tile and never rescaled afterwards (so the
// accumulators are only ever touched by MFMA).  A later tile in which a
// head's weight 2^(logit - reference) could exceed 2^kWideBail (weights up
// to 2^64 are exact in fp32/bf16 range terms) makes the workgroup start
// over with the exact maximum from a first pass over all its rows.  The
// lagged (128-head) loop tests the head's weight sum over the tile, which
// it forms anyway, instead of the tile's maximum; the sum bounds every
// weight, and a large sum of moderate weights only costs an exact restart.
constexpr float kWideBail = 64.f;
// QK steps before the end of a tile's QK at which the lagged loop issues the
// LDS reads of the PV products that follow (their latency then overlaps the
// last QK products)
constexpr int kHookSteps = 4;

// QK products with the accumulator in VGPRs (the compiler gives every MFMA
// of a function the same accumulator file, and O^T fills the accumulator
// registers): dst = srcC (exact overlap; the hardware forwards the
// accumulation chain).  Results are read only after mla_qk_settle.
__device__ __forceinline__ f32x4 mla_qk_first(bf16x8 k, bf16x8 q) {
  f32x4 d;
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "v"(q));
  return d;
}
__device__ __forceinline__ void mla_qk_acc(f32x4& d, bf16x8 k, bf16x8 q) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "v"(q));
}
// Wait states between the last QK product and the first vector-ALU read of
// its result (the compiler does not see inside the instructions above):
// 24 >= the XDL-write-to-VALU-read requirement of an 8-pass MFMA.
__device__ __forceinline__ void mla_qk_settle(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Tile layout of the wide kernel: a 32-row tile is 36 column blocks of
// 1 KB, block c holding bytes [32c, 32c+32) of all 32 rows as two halves
// of 512 bytes (bytes [32c, 32c+16) of every row, then [32c+16, 32c+32));
// within the second half the rows are permuted r -> r ^ 8.  One DMA
// wave-instruction fills exactly one block (lane l lands at 16l: half
// l >> 5, row (l & 31) ^ 8(l >> 5)), so every lane gathers from a single
// row of the tile for all its instructions, and both the K fragment reads
// (16 rows x 16 bytes per 16-lane group) and the transposed V reads (4
// rows x 32 bytes) hit distinct banks.
constexpr int kWideTileBytes = kPipeTile * kMlaRowBytes;         // 36864
constexpr int kWideInst = kWideTileBytes / (kWave * 16);         // 36 blocks
// per-lane byte offset of this lane's 16 bytes of K fragment (key block 0,
// k-step 0); key block kb adds 256, k-step ks adds 2048
__device__ __forceinline__ int wide_koff(int l) {
  const int hh = (l >> 4) & 1;
  return (l >> 5) * 1024 + hh * 512 + ((l & 15) ^ (hh << 3)) * 16;
}
// per-lane byte offset of the transposed V read (rows 4g + (li >> 2), the
// 8-byte piece li & 3 of the 32-byte column block of output columns
// [col0, col0 + 16)); column block +1 adds 1024, rows +16 add 256
__device__ __forceinline__ int wide_voff(int l, int col0) {
  const int li = l & 15, g = l >> 4, hh = (li >> 1) & 1;
  return (col0 >> 4) * 1024 + hh * 512 + ((4 * g + (li >> 2)) ^ (hh << 3)) * 16 + (li & 1) * 8;
}
// tile row whose bytes lane l gathers
__device__ __forceinline__ int wide_gather_slot(int l) { return (l & 31) ^ ((l >> 5) << 3); }

// Keys of a tile that hold selected rows (valid rows are compacted to the
// front, so only the last tile is partial): the first `rem` of 32.
__device__ __forceinline__ uint64_t tile_valid_mask(int32_t rem) {
  return rem >= kPipeTile ? 0xffffffffull : ((1ull << (rem > 0 ? rem : 0)) - 1ull);
}

// The global address a lane gathers from for the DMA instructions of a
// tile: its row (a row of -1 reads row 0; the kernel pads with a selected
// row instead), its half, and the issuing wave's first column block.
// 64-bit per lane, so the latent KV may exceed 4 GiB; the blocks a wave
// issues are kNW * 32 bytes apart.
__device__ __forceinline__ const uint8_t* wide_gather_src(const uint8_t* kv, int32_t row, int l,
                                                          int wave) {
  row = row < 0 ? 0 : row;
  return kv + static_cast<int64_t>(row) * kMlaRowBytes + ((l >> 5) << 4) + 32 * wave;
}
// One DMA wave-instruction: the block at LDS address lds (the block's
// start: lane l lands at lds + 16l) from the lane's address src (bytes
// [32m, 32m+32) of its row for block m).  The instruction's own offset
// field stays 0: for loads into LDS it moves the LDS destination as well
// as the global address, so the block offset is added to src instead.
__device__ __forceinline__ void wide_gather_issue(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}

template <int kNW>
struct MlaWideShared {
  static constexpr int kHeads = 32 * kNW;
  uint4 qrope[2][4][kHeads];   // rope k-steps of Q^T: [ks-16][lane group][head]
  int32_t sidx[kMlaMaxKeys + kPipeTile];   // + one tile of -1: the lagged loop's last gather
  uint4 p[2][4][kHeads];       // P^T fragments: [tile parity][lane group][head] -> 8 bf16
  int32_t wave_cnt[kNW];       // index compaction scratch
  int32_t bail[kNW];           // wave w saw a tile beyond its reference + 2^kWideBail
  float m_fin[kHeads], l_fin[kHeads];
};

template <int kNW, bool kLag>
__global__ void __launch_bounds__(kWave * kNW) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_bf16_wide_kernel(MlaArgs a, int32_t keys_per_split) {
  constexpr int kThreads = kWave * kNW;
  constexpr int kHeads = 32 * kNW;
  constexpr int kHG = kHeads / 16;            // 16-head blocks of PV
  constexpr int kCols = kMlaDl / kNW;         // output columns per wave
  constexpr int kCB = kCols / 16;             // 16-column blocks per wave
  constexpr int kCBC = kCB < 4 ? kCB : 4;     // column blocks per PV chunk
  constexpr int kPer = kWideInst / kNW;      // DMA wave-instructions per wave and tile
  static_assert(kPer * kNW == kWideInst, "the tile's blocks split evenly over the waves");
  constexpr int kQReg = kMlaDl / 32;          // latent k-steps of Q^T in VGPRs (16)
  __shared__ MlaWideShared<kNW> sh;
  // Names an accumulator register so that the compiler places the MFMA
  // accumulators (O^T) in the accumulator file.
  asm volatile("" ::: "a0");

  // Queries in reverse order: in causal prefill the later queries select
  // the most rows, so the longest workgroups start first and the short ones
  // fill the tail.  Split-major ids (decode): the splits of a query are
  // n_q ids apart, so with n_q a multiple of 8 they run on one XCD, whose L2
  // then serves the query's Q to all of them.
  const int32_t jr = blockIdx.x % a.n_q;
  const int32_t split = blockIdx.x / a.n_q;
  const int32_t j = a.n_q - 1 - jr;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int h0 = wave * 32 + li;              // heads h0, h0+16: logits and softmax of this lane

  const int32_t s_begin = split * keys_per_split;
  int32_t s_end = s_begin + keys_per_split;
  s_end = s_end < a.topk ? s_end : a.topk;
  const int32_t n_keys = s_end > s_begin ? s_end - s_begin : 0;
  // Loads first, all in flight together: the selected row indices (every
  // one of the split's, kIdx per thread) and Q^T.  The compaction below
  // then waits only for the indices, and Q lands while it runs.
  const int32_t* idx_row = a.topk_idx + static_cast<int64_t>(j) * a.topk + s_begin;
  constexpr int kIdx = kMlaMaxKeys / kThreads;
  int32_t ridx[kIdx];
#pragma unroll
  for (int it = 0; it < kIdx; ++it) {
    const int32_t i = it * kThreads + tid;
    ridx[it] = i < n_keys ? idx_row[i] : -1;
  }
  // Q^T fragments (B operand of QK) of heads h0 and h0+16: dims 32*ks +
  // 8*grp + 0..7; the latent k-steps in VGPRs, the 2 rope k-steps in LDS
  bf16x8 qf[2][kQReg];
  auto q_of = [&](int hb) {
    return static_cast<const uint16_t*>(a.q) +
           (static_cast<int64_t>(j) * a.n_heads + h0 + 16 * hb) * kMlaD + grp * 8;
  };
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* q = q_of(hb);
#pragma unroll
    for (int ks = 0; ks < kQReg; ++ks)
      qf[hb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + ks * 32));
  }
  // valid row indices, compacted in their given order (ordered ballot
  // scan); LDS-only barriers, so the Q loads stay in flight
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  int32_t n_valid = 0;
#pragma unroll
  for (int it = 0; it < kIdx; ++it) {
    if (it * kThreads >= n_keys) continue;   // uniform
    const int32_t r = ridx[it];
    const bool ok = r >= 0 && r < a.kv_rows;
    const uint64_t ball = __ballot(ok);
    if (lane == 0) sh.wave_cnt[wave] = static_cast<int32_t>(__popcll(ball));
    lds_barrier();
    int32_t before = n_valid, total = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const int32_t c = sh.wave_cnt[w];
      before += w < wave ? c : 0;
      total += c;
    }
    if (ok) sh.sidx[before + __popcll(ball & ((1ull << lane) - 1ull))] = r;
    n_valid += total;
    lds_barrier();
  }
  const int32_t n_tiles = static_cast<int32_t>(ceil_div(n_valid, kPipeTile));
  // Slots past the valid rows (the last tile's tail, and the tile after it
  // that the lagged loop gathers into a free buffer) repeat the last valid
  // row: their logits are masked by position and their softmax weight is 0,
  // but they must hold finite values (0 x NaN would poison PV), and a
  // selected row is the one row the caller guarantees to be initialised.
  const int32_t pad_row = n_valid > 0 ? sh.sidx[n_valid - 1] : 0;
  for (int32_t i = n_valid + tid; i < (n_tiles + 1) * kPipeTile; i += kThreads) sh.sidx[i] = pad_row;
  if (tid < kNW) sh.bail[tid] = 0;
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t* kv = static_cast<const uint8_t*>(a.kv);
  const uint32_t lds_bufs = static_cast<uint32_t>(
      (size_t)((__attribute__((address_space(3))) uint8_t*)g_mla_bufs));
  // wave w issues blocks w, w + kNW, ...: slot i is block kNW*i + wave
  auto slot_lds = [&](int b, int i) {
    return lds_bufs + static_cast<uint32_t>(b * kPipeTileBytes + (kNW * i + wave) * 1024);
  };
  auto row_of = [&](int t0) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return wide_gather_src(kv, sh.sidx[t0 + wide_gather_slot(ln)], ln, wave);
  };
  // all of this wave's slots of the tile with rows sidx[t0..] into buffer b
  auto issue_tile = [&](int b, int t0) {
    const uint8_t* src = row_of(t0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) wide_gather_issue(src + 32 * kNW * i, slot_lds(b, i));
  };
  // The first tile's gather goes out before the rope part of Q is loaded,
  // so that the two latencies overlap (the lagged loop issues it here on its
  // first pass; the padding rows of the index list must be visible first).
  // Then everything lands before the tile loop: the compiler's own waits for
  // Q inside the loop would not account for the gathers.
  lds_barrier();
  if (kLag && n_tiles > 0) issue_tile(0, 0);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int r = 0; r < 2; ++r)
      sh.qrope[r][grp][h0 + 16 * hb] = *reinterpret_cast<const uint4*>(q_of(hb) + (kQReg + r) * 32);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // S^T = K Q^T of the tile in buf for heads h0, h0+16 (2 key blocks x 2
  // head blocks), optionally issuing this wave's gather slots of another
  // tile (rows sidx[t0g..], into gbuf) spread over the k-steps.  `hook`
  // runs after the products of step kMlaKSteps - kHookSteps: the lagged
  // loop issues there the LDS reads of the PV products that follow, so
  // that their latency is spent under the last QK products.
  auto qk = [&](const uint8_t* tile, f32x4 (&st)[2][2], bool gather, int t0g, int gb,
                auto&& hook) __attribute__((always_inline)) {
    // the gather's row is read first, so that waiting for it does not wait
    // for the K fragment reads behind it
    const uint8_t* gsrc = gather ? row_of(t0g) : kv;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int koff = wide_koff(ln);
    auto kfrag = [&](int kb, int ks) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(tile + koff + kb * 256 + ks * 2048));
    };
    // step s multiplies k-step ks_of(s): the two rope k-steps first, whose
    // Q^T fragments come from LDS and are read here with the first K
    // fragments, then the latent ones (Q^T in VGPRs)
    auto ks_of = [](int s) { return s < 2 ? kQReg + s : s - 2; };
    bf16x8 qr[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        qr[r][hb] = __builtin_bit_cast(bf16x8, sh.qrope[r][grp][h0 + 16 * hb]);
    // K fragments are read kAhead steps before their products; the
    // scheduling barriers keep the compiler from sinking the reads next to
    // their use (one wave per SIMD: nothing else hides the LDS latency)
    constexpr int kAhead = 2;
    // steps over which the gather slots are spread.  The lagged schedule
    // gathers only one tile ahead, so its slots go out in the first two
    // thirds: spread wider, the CU's memory queue backs up less behind
    // them (over 9 steps the 9 slots stalled the issue ~530 clocks per
    // tile), while the last one still lands before the tile's barrier
    // (12 against 9 steps: 8000 tokens 490 -> 484 us, 65536-token fp8
    // 4456 -> 4369 us; 18 steps: no consistent gain)
    constexpr int kSpread = kLag ? 12 : kMlaKSteps;
    bf16x8 kf[kAhead + 1][2];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) {
      kf[s][0] = kfrag(0, ks_of(s));
      kf[s][1] = kfrag(1, ks_of(s));
    }
#pragma unroll
    for (int s = 0; s < kMlaKSteps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s + kAhead < kMlaKSteps) {
        kf[(s + kAhead) % (kAhead + 1)][0] = kfrag(0, ks_of(s + kAhead));
        kf[(s + kAhead) % (kAhead + 1)][1] = kfrag(1, ks_of(s + kAhead));
      }
      // the reads go out before this step's products, not after them
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 k0 = kf[s % (kAhead + 1)][0], k1 = kf[s % (kAhead + 1)][1];
      const int ks = ks_of(s);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bf16x8 qv = ks < kQReg ? qf[hb][ks < kQReg ? ks : 0] : qr[ks - kQReg][hb];
        // four independent chains (key block x head block)
        if (s == 0) {
          st[0][hb] = mla_qk_first(k0, qv);
          st[1][hb] = mla_qk_first(k1, qv);
        } else {
          mla_qk_acc(st[0][hb], k0, qv);
          mla_qk_acc(st[1][hb], k1, qv);
        }
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i * kSpread / kPer == s && gather) wide_gather_issue(gsrc + 32 * kNW * i, slot_lds(gb, i));
      }
      if (s == kMlaKSteps - kHookSteps) {
        __builtin_amdgcn_sched_barrier(0);
        hook();
      }
    }
    mla_qk_settle(st[0][0], st[0][1], st[1][0], st[1][1]);
  };
  auto no_hook = []() __attribute__((always_inline)) {};
  // scaled logits, masked: st[kb][hb][i] is key 16kb + 4grp + i, head h0+16hb
  auto logits = [&](f32x4 (&st)[2][2], uint64_t valid, float (&mx)[2]) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb * 16 + grp * 4 + i;
          const float l = ((valid >> key) & 1ull) ? st[kb][hb][i] * scale2 : -INFINITY;
          st[kb][hb][i] = l;
          m = fmaxf(m, l);
        }
      mx[hb] = mla_rows_max(m);
    }
  };

  float m_ref[2] = {-INFINITY, -INFINITY};
  bool exact = false;   // m_ref is the exact maximum (after a restart)
  f32x4 o[kCB][kHG];
  float l_run[2];

  // ---- lagged schedule (kLag): the softmax of tile t runs interleaved
  // with the PV products of tile t-1, so that its vector work (about 600
  // clocks per tile, the 16 exponentials at quarter rate included) issues
  // in the shadow of the matrix core.  One wave per SIMD issues in order
  // and an MFMA holds the next one back for its 16 clocks, so the
  // interleave has to be one product at a time: unit u (of 64) is a small
  // piece of softmax followed by one PV product, with scheduling barriers
  // between them so that the compiler keeps that order.
  //   pv_c: issue the PV products of the previous tile (its V^T fragments
  //         in vf and the P^T fragments of head groups 0 and 1 in pf, read
  //         by pv_reads; the later groups are read two groups ahead from
  //         parity buffer pb_rd); sm_c: run the softmax of st and write its
  //         P^T to parity buffer pb_wr.  Softmax without PV is the first
  //         tile, which also sets the reference maximum.
  constexpr int kCBL = kCB < 8 ? kCB : 8;   // column blocks whose V fragments are held
  bf16x8 vf[kCBL];
  bf16x8 pf[3];
  // P^T fragment reads of the tile's PV products: this lane's address in the
  // parity buffer being read is formed once per tile (by pv_reads); head
  // group hg adds 256 bytes, an instruction offset
  const __attribute__((address_space(3))) uint8_t* p_rd = nullptr;
  auto load_p = [&](int pb, int hg) __attribute__((always_inline)) {
    (void)pb;   // p_rd already points into parity buffer pb
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(p_rd + hg * 256));
  };
  // the LDS reads the PV products of a tile start with: its V^T fragments
  // (transposed reads of the tile in vtile) and P^T of head groups 0 and 1
  auto pv_reads = [&](const uint8_t* vtile, int pb) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    p_rd = (const __attribute__((address_space(3))) uint8_t*)(&sh.p[pb][ln >> 4][ln & 15]);
    const int voff = wide_voff(ln, wave * kCols);
#pragma unroll
    for (int c = 0; c < kCBL; ++c) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vtile + voff + c * 1024));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vtile + voff + 256 + c * 1024));
      vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    pf[0] = load_p(pb, 0);
    pf[1] = load_p(pb, 1);
  };
  auto phase_b = [&](auto pv_c, auto sm_c, int pb_rd, int pb_wr, f32x4 (&st)[2][2],
                     bool& beyond) __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_c)::value;
    constexpr bool kSM = decltype(sm_c)::value;
    constexpr bool kFirst = !kPV;
    constexpr int kUnits = kCB * kHG;         // PV products per tile and wave
    static_assert(kUnits == 64, "64 PV products per tile and wave");
    static_assert(kCB == kCBL, "the lagged schedule holds every V fragment of the wave");
    float mx[2], nm[2], psum[2] = {0.f, 0.f};
    bf16x8 pvb[2];
    // softmax pieces; u is a compile-time constant once the unit loop is
    // unrolled.  Values: st[kb][hb][i] is key 16kb + 4grp + i of head
    // h0 + 16hb; v = 8hb + 4kb + i.
    auto micro = [&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < 4 && !kFirst) {
        // after the first tile the maximum is not needed: a rise past the
        // reference shows in the head's weight sum (unit 55), for fewer
        // vector instructions between the products
      } else if constexpr (u < 2) {                       // raw maximum of head block u
        const float m0 = max3_raw(st[0][u][0], st[0][u][1], st[0][u][2]);
        const float m1 = max3_raw(st[0][u][3], st[1][u][0], st[1][u][1]);
        mx[u] = max3_raw(m0, m1, max_raw(st[1][u][2], st[1][u][3]));
      } else if constexpr (u == 2) {               // across the four 16-lane rows
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const auto a2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[hb]),
                                                            __float_as_uint(mx[hb]), false, false);
          mx[hb] = max_raw(__uint_as_float(a2[0]), __uint_as_float(a2[1]));
        }
      } else if constexpr (u == 3) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const auto b2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx[hb]),
                                                            __float_as_uint(mx[hb]), false, false);
          mx[hb] = max_raw(__uint_as_float(b2[0]), __uint_as_float(b2[1])) * scale2;
        }
      } else if constexpr (u == 4) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          if (kFirst && !exact) m_ref[hb] = mx[hb];
          nm[hb] = -m_ref[hb];
        }
      } else if constexpr (u == 5) {
        if constexpr (kFirst) beyond = false;   // the reference is this tile's maximum
      } else if constexpr (u < 6 + 3 * 16) {       // weights exp2(scale2 * s - m_ref), three steps per value
        constexpr int v = (u - 6) / 3, ph = (u - 6) % 3;
        constexpr int hb = v >> 3, kb = (v >> 2) & 1, i = v & 3;
        if constexpr (ph == 0) {
          st[kb][hb][i] = __builtin_fmaf(st[kb][hb][i], scale2, nm[hb]);
        } else if constexpr (ph == 1) {
          st[kb][hb][i] = __builtin_amdgcn_exp2f(st[kb][hb][i]);
        } else {
          psum[hb] += st[kb][hb][i];
          if constexpr ((i & 1) != 0) {
            pvb[hb][kb * 4 + i - 1] = static_cast<__bf16>(st[kb][hb][i - 1]);
            pvb[hb][kb * 4 + i] = static_cast<__bf16>(st[kb][hb][i]);
          }
        }
      } else if constexpr (u == 54) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const auto a2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum[hb]),
                                                            __float_as_uint(psum[hb]), false, false);
          psum[hb] = __uint_as_float(a2[0]) + __uint_as_float(a2[1]);
        }
      } else if constexpr (u == 55) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const auto b2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(psum[hb]),
                                                            __float_as_uint(psum[hb]), false, false);
          const float tile_sum = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
          l_run[hb] += tile_sum;
          // a weight above 2^kWideBail (or an infinite one) puts the head's
          // tile sum above it; a sum above it without such a weight only
          // costs a restart, which is exact
          static_assert(kWideBail == 64.f, "the bound below is 2^kWideBail");
          if constexpr (!kFirst) beyond = beyond || (!exact && !(tile_sum <= 0x1p64f));
        }
      } else if constexpr (u == 56) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          sh.p[pb_wr][grp][h0 + 16 * hb] = __builtin_bit_cast(uint4, pvb[hb]);
      } else if constexpr (u == 57) {
        if (__ballot(beyond) != 0ull && lane == 0) sh.bail[wave] = 1;
      }
    };
    static_for<kUnits>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (kSM) micro(uc);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kPV) {
        constexpr int hg = u / kCBL, c = u % kCBL;
        // P^T fragments are read two head groups ahead
        if constexpr (c == 0 && hg + 2 < kHG) pf[(hg + 2) % 3] = load_p(pb_rd, hg + 2);
        o[c][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c], pf[hg % 3], o[c][hg], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // At most two passes: the second runs with the exact maximum, against
  // which no tile can rise (its bail test is off), so the loop ends.
  for (int pass = 0; pass < 2; ++pass) {
    if (exact) {
      // ---- first pass: exact maximum of every head over all rows (tiles
      //      gathered one at a time into buffer 0)
      m_ref[0] = m_ref[1] = -INFINITY;
      for (int32_t t = 0; t < n_tiles; ++t) {
        __syncthreads();   // buffer 0 free
        issue_tile(0, t * kPipeTile);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        const uint64_t valid = tile_valid_mask(n_valid - t * kPipeTile);
        f32x4 st[2][2];
        qk(g_mla_bufs, st, false, 0, 0, no_hook);
        float mx[2];
        logits(st, valid, mx);
        m_ref[0] = fmaxf(m_ref[0], mx[0]);
        m_ref[1] = fmaxf(m_ref[1], mx[1]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int hg = 0; hg < kHG; ++hg) o[cb][hg] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run[0] = l_run[1] = 0.f;
    if (n_tiles > 0 && (exact || !kLag)) issue_tile(0, 0);
    if (!kLag && n_tiles > 1) issue_tile(1, kPipeTile);
    bool bailed = false;
    if constexpr (kLag) {
      // tile t lives in buffer t mod 3; its gather was issued during QK of
      // tile t-1.  One barrier per tile: tile t has landed, P^T of tile t-1
      // and the bail flags of its softmax are visible, and every wave is
      // done with PV of tile t-2, whose buffer takes the gather of t+1.
      const std::true_type yes{};
      const std::false_type no{};
      // QK of tile t (buffer b) with the gather of tile t+1 spread through it
      auto qk_tile = [&](int32_t t, int b, f32x4 (&st)[2][2], auto&& hook) __attribute__((always_inline)) {
        const uint8_t* tile = g_mla_bufs + b * kPipeTileBytes;
        // the gather of tile t+1 is issued unconditionally (after the last
        // tile it reads padding rows into a free buffer), so the k-step loop
        // has no branch; the epilogue waits for it before reusing the buffers
        qk(tile, st, true, (t + 1) * kPipeTile, b == 2 ? 0 : b + 1, hook);
        // valid rows are compacted to the front: only the last tile is
        // partial; its missing keys get a logit of -inf (weight 0)
        const int32_t rem = n_valid - t * kPipeTile;
        if (rem < kPipeTile) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (kb * 16 + grp * 4 + i >= rem) st[kb][hb][i] = -INFINITY;
        }
      };
      auto tile_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) lgkmcnt(0): this wave's gather and P^T writes
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      };
      // the first tile (peeled: softmax alone, and it sets the reference)
      if (n_tiles > 0) {
        tile_barrier();
        f32x4 st[2][2];
        qk_tile(0, 0, st, no_hook);
        bool beyond = false;
        phase_b(no, yes, 0, 0, st, beyond);
      }
      for (int32_t t = 1, b = 1; t < n_tiles; ++t, b = b == 2 ? 0 : b + 1) {
        tile_barrier();
        bool bail = false;
#pragma unroll
        for (int w = 0; w < kNW; ++w) bail |= sh.bail[w] != 0;
        if (bail) {
          bailed = true;
          break;
        }
        f32x4 st[2][2];
        // the PV reads of tile t-1 (buffer b-1, P^T parity (t-1) & 1) go out
        // near the end of QK of tile t
        const uint8_t* vtile = g_mla_bufs + (b == 0 ? 2 : b - 1) * kPipeTileBytes;
        const int pb_rd = (t - 1) & 1;
        qk_tile(t, b, st, [&]() __attribute__((always_inline)) { pv_reads(vtile, pb_rd); });
        bool beyond = false;
        phase_b(yes, yes, pb_rd, t & 1, st, beyond);
      }
      if (!bailed && n_tiles > 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        bool bail = false;
#pragma unroll
        for (int w = 0; w < kNW; ++w) bail |= sh.bail[w] != 0;
        if (bail) {
          bailed = true;
        } else {
          f32x4 st[2][2];
          bool beyond = false;
          const int bl = (n_tiles - 1) % 3;
          pv_reads(g_mla_bufs + bl * kPipeTileBytes, (n_tiles - 1) & 1);
          phase_b(yes, no, (n_tiles - 1) & 1, 0, st, beyond);
        }
      }
    } else
    // tile t lives in buffer t mod 3; its gather was issued two tiles ahead
    for (int32_t t = 0, b = 0; t < n_tiles; ++t, b = b == 2 ? 0 : b + 1) {
      if (t + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPer));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();       // tile t complete; tile t-1 consumed
      asm volatile("" ::: "memory");
      const uint8_t* tile = g_mla_bufs + b * kPipeTileBytes;
      const uint64_t valid = tile_valid_mask(n_valid - t * kPipeTile);
      // ---- QK, with the gather of tile t+2 into the buffer of tile t-1
      f32x4 st[2][2];
      qk(tile, st, t + 2 < n_tiles, (t + 2) * kPipeTile, b == 0 ? 2 : b - 1, no_hook);
      // ---- softmax weights relative to the fixed reference
      float mx[2];
      logits(st, valid, mx);
      bool beyond = false;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (t == 0 && !exact) m_ref[hb] = mx[hb];
        beyond |= !exact && mx[hb] > m_ref[hb] + kWideBail;
        float psum = 0.f;
        bf16x8 pv;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pw = valid ? __builtin_amdgcn_exp2f(st[kb][hb][i] - m_ref[hb]) : 0.f;
            psum += pw;
            pv[kb * 4 + i] = static_cast<__bf16>(pw);
          }
        l_run[hb] += mla_rows_sum(psum);
        sh.p[0][grp][h0 + 16 * hb] = __builtin_bit_cast(uint4, pv);
      }
      if (__ballot(beyond) != 0ull && lane == 0) sh.bail[wave] = 1;
      // P of every head and the bail flags visible to all waves; only LDS
      // traffic is waited for (the gathers stay in flight)
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      bool bail = false;
#pragma unroll
      for (int w = 0; w < kNW; ++w) bail |= sh.bail[w] != 0;
      if (bail) {
        bailed = true;
        break;
      }
      // ---- O^T += V^T P^T for this wave's columns, all heads
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int li_t = ln & 15, grp_t = ln >> 4;
      const int voff = wide_voff(ln, wave * kCols);
#pragma unroll
      for (int c0 = 0; c0 < kCB; c0 += kCBC) {
        bf16x8 vf[kCBC];
#pragma unroll
        for (int c = 0; c < kCBC; ++c) {
          const int cb = c0 + c;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(tile + voff + cb * 1024));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(tile + voff + 256 + cb * 1024));
          vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        bf16x8 pf = __builtin_bit_cast(bf16x8, sh.p[0][grp_t][li_t]);
#pragma unroll
        for (int hg = 0; hg < kHG; ++hg) {
          bf16x8 pn = pf;
          if (hg + 1 < kHG) pn = __builtin_bit_cast(bf16x8, sh.p[0][grp_t][(hg + 1) * 16 + li_t]);
#pragma unroll
          for (int c = 0; c < kCBC; ++c)
            o[c0 + c][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c], pf, o[c0 + c][hg], 0, 0, 0);
          pf = pn;
        }
      }
    }
    if (!bailed) break;
    // start over with the exact maximum: drain the gathers in flight first
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (tid < kNW) sh.bail[tid] = 0;
    exact = true;
  }

  // ---- epilogue: owners publish (m, l).  O goes out through the tile
  // buffers (free now), a block of heads at a time, so that the global
  // stores are whole head rows: a lane's own fragments would make every
  // store instruction cover 16 heads x 32 bytes of partly written lines.
  if (lane < 16) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sh.m_fin[h0 + 16 * hb] = m_ref[hb];
      sh.l_fin[h0 + 16 * hb] = l_run[hb];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the lagged loop's last gather (into a tile buffer)
  __syncthreads();   // also: every wave is done with the tile buffers
  const int col0 = wave * kCols + grp * 4;
  auto write_out = [&](auto esz) {
    constexpr int kE = decltype(esz)::value;         // bytes per element: 2 (bf16) or 4
    constexpr int kRowB = kMlaDl * kE;               // one head row of O
    constexpr int kStride = kRowB + 16;              // padded stage row (banks)
    constexpr int kCH0 = kE == 2 ? 64 : 32;
    constexpr int kCH = kCH0 < kHeads ? kCH0 : kHeads;   // heads per block
    static_assert(kCH * kStride <= 3 * kPipeTileBytes, "a block fits in the tile buffers");
    uint8_t* stage = g_mla_bufs;
#pragma unroll
    for (int c = 0; c < kHeads / kCH; ++c) {
#pragma unroll
      for (int hq = 0; hq < kCH / 16; ++hq) {
        const int hg = c * (kCH / 16) + hq;
        float sc = 1.f;   // split partials stay unnormalised
        if (a.n_splits == 1) {
          const float lf = sh.l_fin[hg * 16 + li];
          sc = lf > 0.f ? 1.f / lf : 0.f;
        }
        uint8_t* srow = stage + (hq * 16 + li) * kStride + col0 * kE;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          if constexpr (kE == 2) {
            uint2 pk;
            pk.x = f32_to_bf16_bits(o[cb][hg][0] * sc) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(o[cb][hg][1] * sc)) << 16);
            pk.y = f32_to_bf16_bits(o[cb][hg][2] * sc) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(o[cb][hg][3] * sc)) << 16);
            *reinterpret_cast<uint2*>(srow + cb * 16 * kE) = pk;
          } else {
            *reinterpret_cast<float4*>(srow + cb * 16 * kE) =
                make_float4(o[cb][hg][0] * sc, o[cb][hg][1] * sc, o[cb][hg][2] * sc, o[cb][hg][3] * sc);
          }
        }
      }
      // LDS-only barriers: waiting for the global stores to retire (as a
      // full __syncthreads would) is not needed to reuse the stage
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      constexpr int kPieces = kRowB / 16;   // 16-byte pieces per head row
      // unrolled: all of a thread's LDS reads are issued before its stores
#pragma unroll
      for (int i = tid; i < kCH * kPieces; i += kThreads) {
        const int r = i / kPieces, q = i - r * kPieces;
        const int h = c * kCH + r;
        uint8_t* dst = a.n_splits == 1
                           ? static_cast<uint8_t*>(a.out) +
                                 (static_cast<int64_t>(j) * a.n_heads + h) * kMlaDl * kE
                           : reinterpret_cast<uint8_t*>(mla_partial_o(a, j, split, h));
        *reinterpret_cast<uint4*>(dst + q * 16) =
            *reinterpret_cast<const uint4*>(stage + r * kStride + q * 16);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // the next block reuses the stage
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  };
  if (a.n_splits == 1 && a.out_dtype != DS_BF16) write_out(std::integral_constant<int, 4>{});
  else write_out(std::integral_constant<int, 2>{});
  if (lane < 16) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = h0 + 16 * hb;
      if (a.n_splits == 1) {
        if (a.lse)
          a.lse[static_cast<int64_t>(j) * a.n_heads + h] =
              l_run[hb] > 0.f ? (m_ref[hb] + log2f(l_run[hb])) * kLn2 : -INFINITY;
      } else {
        float* pml = mla_partial_ml(a, j, split, h);
        pml[0] = m_ref[hb];
        pml[1] = l_run[hb];
      }
    }
  }
}


// Merge split partials: one workgroup per (query, 4 heads), 64 threads per
// head, 8 output columns (one 16-byte load per split) per thread.
constexpr int kMlaMaxSplits = 16;   // topk <= 2048 rows, at least 4 tiles per split
constexpr int kMlaCombineHeads = 4;

__global__ void __launch_bounds__(256)
mla_combine_kernel(MlaArgs a) {
  const int32_t j = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t h = blockIdx.y * kMlaCombineHeads + (tid >> 6);
  const int c = (tid & 63) * 8;
  // every split's (m, l) and this thread's eight columns, all loads in flight
  float ms[kMlaMaxSplits], ls[kMlaMaxSplits];
  uint4 v[kMlaMaxSplits];
#pragma unroll
  for (int s = 0; s < kMlaMaxSplits; ++s) {
    if (s < a.n_splits) {
      const float* pml = mla_partial_ml(a, j, s, h);
      ms[s] = pml[0];
      ls[s] = pml[1];
      v[s] = *reinterpret_cast<const uint4*>(mla_partial_o(a, j, s, h) + c);
    } else {
      ms[s] = -INFINITY;
      ls[s] = 0.f;
      v[s] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMlaMaxSplits; ++s) M = fmaxf(M, ms[s]);
  float Lsum = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMlaMaxSplits; ++s) {
    const float wgt = ms[s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
    Lsum += ls[s] * wgt;
    const uint32_t w4[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] = fmaf(bf16_bits_to_f32(static_cast<uint16_t>(w4[k] & 0xffffu)), wgt, acc[2 * k]);
      acc[2 * k + 1] = fmaf(bf16_bits_to_f32(static_cast<uint16_t>(w4[k] >> 16)), wgt, acc[2 * k + 1]);
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int64_t obase = (static_cast<int64_t>(j) * a.n_heads + h) * kMlaDl + c;
  if (a.out_dtype == DS_BF16) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = f32_to_bf16_bits(acc[2 * k] * inv) |
             (static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * k + 1] * inv)) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + obase) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    float* out = static_cast<float*>(a.out) + obase;
    *reinterpret_cast<float4*>(out) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (a.lse && (tid & 63) == 0)
    a.lse[static_cast<int64_t>(j) * a.n_heads + h] =
        Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host
// fp8 rows -> bf16 rows of code * scale (round to nearest even), 16 codes
// per thread: one 16-byte load, two 16-byte stores.
__global__ void __launch_bounds__(256)
widen_fp8_rows_kernel(const uint8_t* codes, const float* scale, int32_t scale_shift, int64_t rows,
                      uint16_t* out) {
  constexpr int kPer = kMlaD / 16;   // 36 pieces of 16 codes per row
  const int64_t piece = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (piece >= rows * kPer) return;
  const int64_t r = piece / kPer;
  const float sc = scale[r >> scale_shift];
  const uint4 v = *reinterpret_cast<const uint4*>(codes + piece * 16);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float2 lo = fp8x2_to_f32<false>(w[k]);
    const float2 hi = fp8x2_to_f32<true>(w[k]);
    o[2 * k] = f32_to_bf16_bits(lo.x * sc) | (static_cast<uint32_t>(f32_to_bf16_bits(lo.y * sc)) << 16);
    o[2 * k + 1] = f32_to_bf16_bits(hi.x * sc) | (static_cast<uint32_t>(f32_to_bf16_bits(hi.y * sc)) << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(out + piece * 16);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

ds_status launch_widen_fp8_rows(const void* codes, const float* scale, int32_t scale_shift,
                                int64_t rows, void* out, hipStream_t s) {
  if (rows <= 0) return DS_OK;
  const int64_t pieces = rows * (kMlaD / 16);
  widen_fp8_rows_kernel<<<static_cast<unsigned>(ceil_div(pieces, 256)), 256, 0, s>>>(
      static_cast<const uint8_t*>(codes), scale, scale_shift, rows, static_cast<uint16_t*>(out));
  return check_launch("sparse_mla (fp8 rows to bf16)");
}

int32_t mla_decode_splits(int32_t n_q, int32_t topk) {
  // enough workgroups to cover the compute units; at least 4 tiles per split
  const int32_t tiles = static_cast<int32_t>(ceil_div(topk, kMlaTile));
  int32_t want = static_cast<int32_t>(ceil_div(device_cu_count(), n_q > 0 ? n_q : 1));
  int32_t max_splits = tiles / 4 > 0 ? tiles / 4 : 1;
  max_splits = max_splits < kMlaMaxSplits ? max_splits : kMlaMaxSplits;   // the combine's bound
  want = want < max_splits ? want : max_splits;
  return want > 0 ? want : 1;
}

size_t mla_partials_bytes(int32_t n_q, int32_t n_heads, int32_t d_latent,
                          int32_t n_splits) {
  (void)d_latent;   // the kernels that split handle d_latent == kMlaDl only
  return mla_partial_o_bytes(n_q, n_splits, n_heads) +
         sizeof(float) * 2 * static_cast<size_t>(n_q) * n_splits * n_heads;
}

ds_status launch_sparse_mla(const MlaArgs& a, hipStream_t s) {
  if (a.n_q == 0) return DS_OK;
  if (a.q_dtype == DS_F32) {
    const int D = a.d_latent + a.d_rope;
    const size_t smem = sizeof(float) * (D + a.topk) + sizeof(int32_t) * a.topk;
    dim3 grid(a.n_q, a.n_heads);
    mla_f32_kernel<<<grid, 256, smem, s>>>(a);
    return check_launch("sparse_mla (f32)");
  }
  const int32_t per_split =
      static_cast<int32_t>(round_up(ceil_div(a.topk, a.n_splits), kMlaTile));
  const int64_t blocks = static_cast<int64_t>(a.n_q) * a.n_splits;
  if (a.kv_dtype == DS_BF16) {
    switch (a.n_heads) {
      case 32: mla_bf16_wide_kernel<1, false><<<blocks, kWave * 1, 0, s>>>(a, per_split); break;
      case 64: mla_bf16_wide_kernel<2, false><<<blocks, kWave * 2, 0, s>>>(a, per_split); break;
      default: mla_bf16_wide_kernel<4, true><<<blocks, kWave * 4, 0, s>>>(a, per_split);
    }
  } else {   // fp8 codes with per-row or per-block scales (decode)
    mla_fp8_kernel<<<blocks, kWave * (a.n_heads / 16), 0, s>>>(a, per_split);
  }
  ds_status st = check_launch("sparse_mla");
  if (st != DS_OK || a.n_splits == 1) return st;
  dim3 cgrid(a.n_q, a.n_heads / kMlaCombineHeads);
  mla_combine_kernel<<<cgrid, 256, 0, s>>>(a);
  return check_launch("sparse_mla combine");
}

}  // namespace ds32cp
