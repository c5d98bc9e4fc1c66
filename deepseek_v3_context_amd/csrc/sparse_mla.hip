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
// bf16/fp8 path (d_latent 512, d_rope 64, heads a multiple of 32): one
// workgroup per (query, split of its selected rows) with one wave per 32
// heads (two groups of 16 that share every K and V fragment read).  The selected rows are gathered 64 at a time into LDS (one copy
// serves all heads, as key for QK and as value for PV), and every wave runs
// a flash-style loop with MFMA v_mfma_f32_16x16x32_bf16:
//   S^T[key, head] = K[key, :] . Q[head, :]     A = K (LDS), B = Q (regs)
//   O^T[c, head]  += V^T[c, key] . P^T[key, head]
// The transposed form makes the QK output layout (one head per lane, four
// keys per lane) exactly the B operand layout PV needs, so P never leaves
// registers; O^T (2 x 16 heads x 512) stays in 256 accumulator registers
// per lane and each lane owns one head per group, so the online-softmax
// rescale is one scalar per lane and group.  fp8 rows are widened to bf16 exactly in LDS and their
// per-block scale multiplies the logits of that key and its softmax weight
// before PV (both in fp32).
//
// Decode (few queries) splits each query's selected rows over several
// workgroups that write unnormalised partial outputs with their running
// max and sum; a combine kernel merges them by log-sum-exp.
#include <stdlib.h>

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

// Lazy rescaling: the running reference max of a head only moves when a
// tile's max exceeds it by more than 2^kRescaleLog2, so that exp2 of any
// logit minus the reference stays below 2^8 and the 256-register output
// accumulator is rescaled only on the rare tiles that raise the max.
constexpr float kRescaleLog2 = 8.f;

// 16-head groups per wave.
#ifndef DS32CP_MLA_GROUPS
#define DS32CP_MLA_GROUPS 1
#endif
constexpr int kMlaGroups = DS32CP_MLA_GROUPS;

template <bool kFp8, bool kTrV, int kG>
__global__ void __launch_bounds__(kWave * 8 / kG)
mla_mfma_kernel(MlaArgs a, int32_t keys_per_split) {
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
  // this lane's heads: one per 16-head group of the wave
  const int hbase = wave * 16 * kG + (lane & 15);

  const int32_t s_begin = split * keys_per_split;
  int32_t s_end = s_begin + keys_per_split;
  s_end = s_end < a.topk ? s_end : a.topk;

  // Q^T fragments (B operand): head h, dims 32*ks + 8*grp + 0..7.
  bf16x8 qf[kG][kMlaKSteps];
#pragma unroll
  for (int g2 = 0; g2 < kG; ++g2) {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<int64_t>(j) * a.n_heads + hbase + 16 * g2) * kMlaD + grp * 8;
#pragma unroll
    for (int ks = 0; ks < kMlaKSteps; ++ks)
      qf[g2][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + ks * 32));
  }

  f32x4 o[kG][kMlaCBlocks];
  float m_ref[kG];   // reference max (log2 domain)
  float l_run[kG];   // sum of exp2(logit - m_ref)
#pragma unroll
  for (int g2 = 0; g2 < kG; ++g2) {
    m_ref[g2] = -INFINITY;
    l_run[g2] = 0.f;
#pragma unroll
    for (int cb = 0; cb < kMlaCBlocks; ++cb) o[g2][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float scale2 = a.sm_scale * kLog2e;

  for (int32_t t0 = s_begin; t0 < s_end; t0 += kMlaTile) {
    // ---- gather the tile's rows into LDS
    if (tid < kMlaTile) {
      const int32_t s = t0 + tid;
      int32_t r = s < s_end ? a.topk_idx[static_cast<int64_t>(j) * a.topk + s] : -1;
      if (r >= a.kv_rows) r = -1;
      rows[tid] = r;
      kscale[tid] = (kFp8 && r >= 0) ? a.kv_scale[r / kFp8BlockRows] : 1.f;
      const uint64_t b = __ballot(r >= 0);
      if (tid == 0) any_valid = b != 0ull;
    }
    __syncthreads();
    if (!any_valid) {
      __syncthreads();
      continue;
    }
    if constexpr (kFp8) {
      constexpr int kPieces = kMlaTile * (kMlaD / 16);   // 16 codes per piece
      for (int piece = tid; piece < kPieces; piece += nthreads) {
        const int r = piece / (kMlaD / 16);
        const int c8 = piece - r * (kMlaD / 16);
        const int32_t row = rows[r];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row >= 0)
          v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.kv) +
                                              static_cast<int64_t>(row) * kMlaD + c8 * 16);
        const uint2 a0 = fp8x4_to_bf16x4(v.x), a1 = fp8x4_to_bf16x4(v.y);
        const uint2 a2 = fp8x4_to_bf16x4(v.z), a3 = fp8x4_to_bf16x4(v.w);
        *reinterpret_cast<uint4*>(&tile[tile_off(r, 2 * c8)]) = make_uint4(a0.x, a0.y, a1.x, a1.y);
        *reinterpret_cast<uint4*>(&tile[tile_off(r, 2 * c8 + 1)]) = make_uint4(a2.x, a2.y, a3.x, a3.y);
      }
    } else {
      constexpr int kPieces = kMlaTile * kMlaRowChunks;
      for (int piece = tid; piece < kPieces; piece += nthreads) {
        const int r = piece / kMlaRowChunks;
        const int c = piece - r * kMlaRowChunks;
        const int32_t row = rows[r];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row >= 0)
          v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.kv) +
                                              static_cast<int64_t>(row) * kMlaRowBytes + c * 16);
        *reinterpret_cast<uint4*>(&tile[tile_off(r, c)]) = v;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for 4 blocks of 16 keys, both head groups
    f32x4 st[kG][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int g2 = 0; g2 < kG; ++g2) st[g2][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = kb * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < kMlaKSteps; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&tile[tile_off(r, ks * 4 + grp)]));
#pragma unroll
        for (int g2 = 0; g2 < kG; ++g2)
          st[g2][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[g2][ks], st[g2][kb], 0, 0, 0);
      }
    }

    // ---- online softmax; this lane: one head per group, keys 16*kb + 4*grp + i
    bf16x8 pb[kG][2];
#pragma unroll
    for (int g2 = 0; g2 < kG; ++g2) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb * 16 + grp * 4 + i;
          float l = st[g2][kb][i] * scale2;
          if constexpr (kFp8) l *= kscale[key];
          l = rows[key] >= 0 ? l : -INFINITY;
          st[g2][kb][i] = l;
          mx = fmaxf(mx, l);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // move the reference only when needed (uniform over the wave)
      const bool need = mx > m_ref[g2] + kRescaleLog2;
      if (__ballot(need)) {
        const float m_new = need ? mx : m_ref[g2];
        const float alpha = __builtin_amdgcn_exp2f(m_ref[g2] - m_new);   // 0 when m_ref = -inf
        l_run[g2] *= alpha;
#pragma unroll
        for (int cb = 0; cb < kMlaCBlocks; ++cb) o[g2][cb] *= alpha;
        m_ref[g2] = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = __builtin_amdgcn_exp2f(st[g2][kb][i] - m_ref[g2]);
          psum += p;
          if constexpr (kFp8) p *= kscale[kb * 16 + grp * 4 + i];   // fold row scale into P
          pb[g2][kb >> 1][(kb & 1) * 4 + i] = static_cast<__bf16>(p);
        }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run[g2] += psum;
    }

    // ---- O^T += V^T P^T, two steps of 32 keys; one V fragment feeds both
    //      head groups
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int r0 = (2 * kp) * 16 + grp * 4;       // keys r0..r0+3
      const int r1 = (2 * kp + 1) * 16 + grp * 4;   // keys r1..r1+3
#pragma unroll
      for (int cb = 0; cb < kMlaCBlocks; ++cb) {
        bf16x8 vf;
        if constexpr (kTrV) {
          // ds_read_b64_tr_b16: in each 16-lane group, lane i names 4
          // consecutive bf16 of row (base + i/4), columns 4*(i%4)..+3 of
          // the 16-column block; lane i receives column i of the 4 rows.
          const int li = lane & 15;
          const int chunk = 2 * cb + ((li & 3) >> 1);
          const int sub = (li & 1) * 8;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(&tile[tile_off(r0 + (li >> 2), chunk) + sub]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(&tile[tile_off(r1 + (li >> 2), chunk) + sub]));
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          vf = __builtin_bit_cast(bf16x8, both);
        } else {
          const int c = cb * 16 + (lane & 15);        // value column
          const int chunk = c >> 3;
          const int within = (c & 7) * 2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vf[i] = *reinterpret_cast<const __bf16*>(&tile[tile_off(r0 + i, chunk) + within]);
            vf[4 + i] = *reinterpret_cast<const __bf16*>(&tile[tile_off(r1 + i, chunk) + within]);
          }
        }
#pragma unroll
        for (int g2 = 0; g2 < kG; ++g2)
          o[g2][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[g2][kp], o[g2][cb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int g2 = 0; g2 < kG; ++g2) {
    const int h = hbase + 16 * g2;
    if (a.n_splits == 1) {
      const float inv = l_run[g2] > 0.f ? 1.f / l_run[g2] : 0.f;
      const int64_t obase = (static_cast<int64_t>(j) * a.n_heads + h) * kMlaDl + grp * 4;
      if (a.out_dtype == DS_BF16) {
        uint16_t* out = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
        for (int cb = 0; cb < kMlaCBlocks; ++cb) {
          uint2 pk;
          pk.x = f32_to_bf16_bits(o[g2][cb][0] * inv) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(o[g2][cb][1] * inv)) << 16);
          pk.y = f32_to_bf16_bits(o[g2][cb][2] * inv) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(o[g2][cb][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(out + cb * 16) = pk;
        }
      } else {
        float* out = static_cast<float*>(a.out) + obase;
#pragma unroll
        for (int cb = 0; cb < kMlaCBlocks; ++cb)
          *reinterpret_cast<float4*>(out + cb * 16) =
              make_float4(o[g2][cb][0] * inv, o[g2][cb][1] * inv, o[g2][cb][2] * inv,
                          o[g2][cb][3] * inv);
      }
      if (a.lse && grp == 0)
        a.lse[static_cast<int64_t>(j) * a.n_heads + h] =
            l_run[g2] > 0.f ? (m_ref[g2] + log2f(l_run[g2])) * kLn2 : -INFINITY;
    } else {
      uint16_t* po = mla_partial_o(a, j, split, h) + grp * 4;
#pragma unroll
      for (int cb = 0; cb < kMlaCBlocks; ++cb)
        mla_store_bf16x4(po + cb * 16, o[g2][cb][0], o[g2][cb][1], o[g2][cb][2], o[g2][cb][3]);
      if (grp == 0) {
        float* pml = mla_partial_ml(a, j, split, h);
        pml[0] = m_ref[g2];
        pml[1] = l_run[g2];
      }
    }
  }
}

// ------------------------------------------------- bf16 KV, pipelined
// One workgroup of 2*kG waves (kG = n_heads/32) per (query, split of its
// rows), in two groups of kG waves; group g owns heads [g*H/2, (g+1)*H/2).
//   * QK + softmax: wave wg of group g owns 16 heads, g*H/2 + 16*wg + 0..15.
//     S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with K from LDS and Q^T (72
//     VGPRs) in registers; the online softmax of a head lives in the lane
//     group that owns it.  The bf16 softmax weights P go to LDS.
//   * PV: wave wg owns output columns [wg*512/kG, (wg+1)*512/kG) of its
//     group's heads: O^T[c, h] += V^T[c, key] P^T[key, h], so each V
//     fragment (LDS transpose read) feeds kG MFMAs.  O^T is 128 fp32
//     registers per lane.
//   * Ping-pong: group 1 runs one phase behind group 0 (an extra barrier
//     before its loop), so while one group does QK + softmax of tile t (LDS
//     reads of K, exp on the vector ALU) the other does PV of its previous
//     tile (MFMA-dense) on the same SIMDs.  Each tile lives in LDS for three
//     phases, so tiles are triple-buffered.
// 32-row tiles are gathered straight into LDS (global_load_lds_dwordx4, no
// VGPRs) by group 0 during its PV phase, two tiles ahead.
// Lazy rescaling: a head's reference max moves only when a tile raises it
// by more than 2^kRescaleLog2; the owner publishes the factor and every
// wave of the group rescales its columns of that head.
constexpr int kPipeTile = 32;                                     // rows per tile
// Padded LDS row of the pipelined kernel: 1184 bytes (74 chunks).  With
// this stride both the K-fragment reads (16 rows, one chunk) and the V
// transpose reads (4 rows x 32 bytes per 16-lane group) are free of bank
// conflicts (measured: 1152 is 4x and 1168 1.5x slower for one of them),
// and a 32-row tile is exactly 37 DMA wave-instructions.
constexpr int kPipeRow = kMlaRowBytes + 32;
constexpr int kDmaRowChunks = kPipeRow / 16;                      // 74 (72 + pad)
constexpr int kPipeTileChunks = kPipeTile * kDmaRowChunks;        // 2368
constexpr int kPipeTileInst = kPipeTileChunks / kWave;            // 37
constexpr int kMlaMaxKeys = 2048;

// Three tile buffers.  The gathers into them are issued as instructions the
// compiler does not see (mla_gather_issue), so it inserts no wait for them
// before reading a buffer; the kernel waits for its gathers itself (vmcnt
// before the barrier that opens a tile).
constexpr int kPipeTileBytes = kPipeTile * kPipeRow;              // 37888
__shared__ __align__(16) uint8_t g_mla_bufs[3 * kPipeTileBytes];

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

// DMA wave-instructions per wave and tile when kW waves share a tile's
// gather (every wave issues the same count; slots past the last
// instruction repeat the wave's previous one: identical bytes to the same
// place).
template <int kW>
struct MlaIssue {
  static constexpr int kPer = (kPipeTileInst + kW - 1) / kW;
};
constexpr int kMlaIssueMax = kPipeTileInst;

template <int kW>
__device__ __forceinline__ int mla_gather_inst(int wave, int i) {
  const int m = wave + i * kW;
  return m < kPipeTileInst ? m : m - kW;
}

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

// One DMA wave-instruction of a tile gather: instruction m fills LDS
// chunks [64m, 64m+64); lane l's chunk is row (64m+l)/74, column
// (64m+l)%74 (columns 72, 73 are padding and re-read column 71).  Empty
// slots (-1) read row 0: their logits are masked and their softmax weight
// is 0.  The lane id is made opaque so this per-lane arithmetic is
// recomputed at every call instead of being hoisted out of the tile loop:
// hoisted values get spilled, and a scratch reload between two DMA
// instructions would wait for the earlier gather (vmcnt counts both).
__device__ __forceinline__ int mla_gather_row(int m, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  return (m * kWave + ln) / kDmaRowChunks;
}

__device__ __forceinline__ void mla_gather_issue(const uint8_t* kv, uint8_t* buf, int m, int lane,
                                                 int32_t row) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int P = m * kWave + ln;
  const int c = P - (P / kDmaRowChunks) * kDmaRowChunks;
  const int cc = c < kMlaRowChunks ? c : kMlaRowChunks - 1;
  row = row < 0 ? 0 : row;
  const uint8_t* src = kv + static_cast<int64_t>(row) * kMlaRowBytes + cc * 16;
  // LDS destination of lane l: M0 + 16*l (M0 = this instruction's chunk
  // block, the same for the whole wave); one wait state between writing M0
  // and the instruction that reads it
  const uint32_t dst = static_cast<uint32_t>(
      (size_t)((__attribute__((address_space(3))) uint8_t*)(buf + m * kWave * 16)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(dst))
               : "memory", "m0");
}

// This wave's slots of the gather of tile rows sidx[t0 .. t0+31] into buf
// (row indices read first: one LDS round trip).
template <int kW>
__device__ __forceinline__ void mla_issue_tile(const uint8_t* kv, uint8_t* buf, const int32_t* sidx,
                                               int t0, int wave, int lane) {
  constexpr int kPer = MlaIssue<kW>::kPer;
  int32_t row[kMlaIssueMax];
#pragma unroll
  for (int i = 0; i < kPer; ++i) row[i] = sidx[t0 + mla_gather_row(mla_gather_inst<kW>(wave, i), lane)];
#pragma unroll
  for (int i = 0; i < kPer; ++i) mla_gather_issue(kv, buf, mla_gather_inst<kW>(wave, i), lane, row[i]);
}

template <int kG>
struct MlaShared {
  static constexpr int kHeads = 32 * kG;
  static constexpr int kHalf = 16 * kG;   // heads per group
  uint4 qrope[2][4][kHeads];   // rope k-steps of Q^T: [ks-16][lane group][head]
  int32_t sidx[kMlaMaxKeys];
  uint4 p[2][4][kHalf];        // P^T fragments: [group][lane group][head in group]
  float alpha[2][kHalf];       // per-tile rescale factor of each head
  int32_t rescale[2][kG];      // wave wg of group g raised a reference max
  int32_t wave_cnt[2 * kG];    // index compaction scratch
  float m_fin[kHeads], l_fin[kHeads];
};

template <bool kTrV, int kG>
__global__ void __launch_bounds__(kWave * 2 * kG)
mla_bf16_pipelined_kernel(MlaArgs a, int32_t keys_per_split) {
  constexpr int kW = 2 * kG;
  constexpr int kThreads = kWave * kW;
  constexpr int kHalf = 16 * kG;              // heads per group
  constexpr int kCols = kMlaDl / kG;          // output columns per wave
  constexpr int kCB = kCols / 16;             // 16-column blocks per wave
  constexpr int kCBC = kCB < 4 ? kCB : 4;     // column blocks per PV chunk
  constexpr int kPer = MlaIssue<kW>::kPer;    // DMA wave-instructions per wave and tile
  __shared__ MlaShared<kG> sh;

  const int32_t j = blockIdx.x / a.n_splits;
  const int32_t split = blockIdx.x - j * a.n_splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave / kG;                    // group
  const int wg = wave - g * kG;               // wave within the group
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int hq = wg * 16 + li;                // head (within the group) this lane keeps
  const int h_own = g * kHalf + hq;

  const int32_t s_begin = split * keys_per_split;
  int32_t s_end = s_begin + keys_per_split;
  s_end = s_end < a.topk ? s_end : a.topk;
  const int32_t n_keys = s_end > s_begin ? s_end - s_begin : 0;
  // Stage the split's valid row indices in LDS, compacted to the front in
  // their given order (ordered ballot scan), so empty slots cost no tiles.
  const int32_t* idx_row = a.topk_idx + static_cast<int64_t>(j) * a.topk + s_begin;
  int32_t n_valid = 0;
  for (int32_t i0 = 0; i0 < n_keys; i0 += kThreads) {
    const int32_t i = i0 + tid;
    const int32_t r = i < n_keys ? idx_row[i] : -1;
    const bool ok = r >= 0 && r < a.kv_rows;
    const uint64_t ball = __ballot(ok);
    if (lane == 0) sh.wave_cnt[wave] = static_cast<int32_t>(__popcll(ball));
    __syncthreads();
    int32_t before = n_valid, total = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const int32_t c = sh.wave_cnt[w];
      before += w < wave ? c : 0;
      total += c;
    }
    if (ok) sh.sidx[before + __popcll(ball & ((1ull << lane) - 1ull))] = r;
    n_valid += total;
    __syncthreads();
  }
  const int32_t n_tiles = static_cast<int32_t>(ceil_div(n_valid, kPipeTile));
  for (int32_t i = n_valid + tid; i < n_tiles * kPipeTile; i += kThreads) sh.sidx[i] = -1;

  // Q^T fragments (B operand of QK): head h_own, dims 32*ks + 8*grp + 0..7;
  // the 16 latent k-steps stay in VGPRs, the 2 rope k-steps in LDS (this
  // keeps the wave clear of register spills, whose scratch reloads would
  // also wait on the in-flight tile gathers)
  constexpr int kQReg = kMlaDl / 32;   // 16
  bf16x8 qf[kQReg];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<int64_t>(j) * a.n_heads + h_own) * kMlaD + grp * 8;
#pragma unroll
    for (int ks = 0; ks < kQReg; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + ks * 32));
#pragma unroll
    for (int r = 0; r < 2; ++r)
      sh.qrope[r][grp][h_own] = *reinterpret_cast<const uint4*>(q + (kQReg + r) * 32);
  }
  // O^T[c, h]: column block cb of this wave, head block hg of the group
  // (head g*H/2 + hg*16 + li, columns 16*cb + 4*grp + 0..3 of this wave's
  // range)
  f32x4 o[kCB][kG];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int hg = 0; hg < kG; ++hg) o[cb][hg] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t* kv = static_cast<const uint8_t*>(a.kv);
  // Q loads complete here, before any gather is in flight: a wait for them
  // inside the tile loop would also wait for the gathers
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();   // sidx and rope ready
  // Gathers: every wave issues its slots of tile t+2 while tile t is in
  // use (group 0 during its PV(t), group 1 during its QK(t); both into the
  // buffer of tile t-1, which both groups have finished with by then), and
  // waits for its slots of a tile before the barrier after which group 0
  // opens it (group 0: the tile-opening barrier; group 1, one phase
  // behind: the P barrier of the step before).  Here: tiles 0 and 1.
  if (n_tiles > 0) mla_issue_tile<kW>(kv, g_mla_bufs, sh.sidx, 0, wave, lane);
  if (n_tiles > 1) mla_issue_tile<kW>(kv, g_mla_bufs + kPipeTileBytes, sh.sidx, kPipeTile, wave, lane);
  if (g == 1) {
    // group 1 runs one phase behind; its part of tile 0 lands before
    // group 0 opens it
    if (n_tiles > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPer));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // tile t lives in buffer t mod 3
  for (int32_t t = 0, b = 0; t < n_tiles; ++t, b = b == 2 ? 0 : b + 1) {
    // this wave's gather of tile t landed (tile t+1 may still be in flight)
    if (g == 0) {
      // group 0's slots of tile t landed (those of tile t+1 may be in flight)
      if (t + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPer));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();         // tile t complete for every wave
    asm volatile("" ::: "memory");
    // QK and softmax are this SIMD's critical path: issue ahead of the
    // other group's PV products
    __builtin_amdgcn_s_setprio(2);
    // tile t+2 goes into the buffer of tile t-1
    const bool gather = t + 2 < n_tiles;
    uint8_t* gbuf = g_mla_bufs + (b == 0 ? 2 : b - 1) * kPipeTileBytes;
    const int t0g = (t + 2) * kPipeTile;
    // row index of this wave's next gather slot, read one slot ahead
    int32_t grow = (g == 1 && gather) ? sh.sidx[t0g + mla_gather_row(mla_gather_inst<kW>(wave, 0), lane)] : 0;
    const uint8_t* tile = g_mla_bufs + b * kPipeTileBytes;
    // per-lane offsets recomputed every tile from an opaque copy of the lane
    // id: hoisted out of the loop they would be spilled
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int li_t = ln & 15, grp_t = ln >> 4;
    const int32_t my_row = lane < kPipeTile ? sh.sidx[t * kPipeTile + lane] : -1;
    const uint64_t valid = __ballot(my_row >= 0);

    // ---- S^T = K Q^T for this wave's 16 heads: 2 blocks of 16 keys; the
    //      fragments of k-step ks+1 are read while ks is multiplied
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const int koff = li_t * kPipeRow + grp_t * 16;
    auto kfrag = [&](int kb, int ks) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(tile + koff + kb * 16 * kPipeRow + ks * 64));
    };
    bf16x8 k0 = kfrag(0, 0), k1 = kfrag(1, 0);
#pragma unroll
    for (int ks = 0; ks < kMlaKSteps; ++ks) {
      bf16x8 n0 = k0, n1 = k1;
      if (ks + 1 < kMlaKSteps) {
        n0 = kfrag(0, ks + 1);
        n1 = kfrag(1, ks + 1);
      }
      const bf16x8 qv = ks < kQReg ? qf[ks < kQReg ? ks : 0]
                                   : __builtin_bit_cast(bf16x8, sh.qrope[ks - kQReg][grp][h_own]);
      st[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qv, st[0], 0, 0, 0);
      st[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qv, st[1], 0, 0, 0);
      k0 = n0;
      k1 = n1;
      // group 1: this wave's gather slots of tile t+2, spread over the k-steps
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i * kMlaKSteps / kPer == ks && g == 1 && gather) {
          mla_gather_issue(kv, gbuf, mla_gather_inst<kW>(wave, i), lane, grow);
          if (i + 1 < kPer) grow = sh.sidx[t0g + mla_gather_row(mla_gather_inst<kW>(wave, i + 1), lane)];
        }
      }
    }
    // ---- online softmax of head h_own over keys 16*kb + 4*grp + i
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb * 16 + grp * 4 + i;
        const float l = ((valid >> key) & 1ull) ? st[kb][i] * scale2 : -INFINITY;
        st[kb][i] = l;
        mx = fmaxf(mx, l);
      }
    mx = mla_rows_max(mx);
    const bool need = mx > m_ref + kRescaleLog2;
    float alpha = 1.f;
    if (need) {
      alpha = __builtin_amdgcn_exp2f(m_ref - mx);   // 0 on the first raise (m_ref = -inf)
      m_ref = mx;
      l_run *= alpha;
    }
    const bool wave_rescales = __ballot(need) != 0ull;
    if (lane < 16) sh.alpha[g][hq] = alpha;
    if (lane == 0) sh.rescale[g][wg] = wave_rescales;
    float psum = 0.f;
    bf16x8 pv;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pw = valid ? __builtin_amdgcn_exp2f(st[kb][i] - m_ref) : 0.f;
        psum += pw;
        pv[kb * 4 + i] = static_cast<__bf16>(pw);
      }
    psum = mla_rows_sum(psum);
    l_run += psum;
    sh.p[g][grp][hq] = __builtin_bit_cast(uint4, pv);
    // P and the rescale factors of the group visible to all its waves.
    // Only LDS traffic is waited for: a fenced barrier would also wait for
    // the tile gathers in flight.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    if (g == 1) {
      // group 1's slots of tile t+1 landed before group 0 opens it after
      // this barrier (those of tile t+2 may be in flight)
      if (gather) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPer));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(0);
    // group 0: its gather slots of tile t+2 go out spread over the products
    if (g == 0 && gather) grow = sh.sidx[t0g + mla_gather_row(mla_gather_inst<kW>(wave, 0), lane)];

    // ---- rescale this wave's columns of any head whose reference moved
    bool any = false;
#pragma unroll
    for (int w = 0; w < kG; ++w) any |= sh.rescale[g][w] != 0;
    if (any) {
#pragma unroll
      for (int hg = 0; hg < kG; ++hg) {
        const float al = sh.alpha[g][hg * 16 + li];
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) o[cb][hg] *= al;
      }
    }
    // ---- O^T += V^T P^T for this wave's column blocks, the group's heads
    const int voff = (4 * grp_t + (li_t >> 2)) * kPipeRow + ((li_t & 3) >> 1) * 16 +
                     (li_t & 1) * 8 + wg * kCols * 2;
    // column blocks in chunks of kCBC: the chunk's V^T fragments stay in
    // registers while every head block of P multiplies them
#pragma unroll
    for (int c0 = 0; c0 < kCB; c0 += kCBC) {
      bf16x8 vf[kCBC];
#pragma unroll
      for (int c = 0; c < kCBC; ++c) {
        const int cb = c0 + c;
        if constexpr (kTrV) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(tile + voff + cb * 32));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(tile + voff + 16 * kPipeRow + cb * 32));
          vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          const int col = wg * kCols + cb * 16 + li;
          const uint8_t* p0 = tile + 4 * grp * kPipeRow + (col >> 3) * 16 + (col & 7) * 2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vf[c][i] = *reinterpret_cast<const __bf16*>(p0 + i * kPipeRow);
            vf[c][4 + i] = *reinterpret_cast<const __bf16*>(p0 + (16 + i) * kPipeRow);
          }
        }
      }
      bf16x8 pf = __builtin_bit_cast(bf16x8, sh.p[g][grp][li]);
#pragma unroll
      for (int hg = 0; hg < kG; ++hg) {
        bf16x8 pn = pf;
        if (hg + 1 < kG) pn = __builtin_bit_cast(bf16x8, sh.p[g][grp][(hg + 1) * 16 + li]);
#pragma unroll
        for (int c = 0; c < kCBC; ++c) {
          o[c0 + c][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c], pf, o[c0 + c][hg], 0, 0, 0);
          const int prod = c0 * kG + hg * kCBC + c;
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            if (i * kG * kCB / kPer == prod && g == 0 && gather) {
              mla_gather_issue(kv, gbuf, mla_gather_inst<kW>(wave, i), lane, grow);
              if (i + 1 < kPer)
                grow = sh.sidx[t0g + mla_gather_row(mla_gather_inst<kW>(wave, i + 1), lane)];
            }
          }
        }
        pf = pn;
      }
    }
  }
  if (g == 0) __builtin_amdgcn_s_barrier();   // pairs with group 1's leading barrier

  // ---- epilogue: owners publish (m, l); every wave writes its columns
  if (lane < 16) {
    sh.m_fin[h_own] = m_ref;
    sh.l_fin[h_own] = l_run;
  }
  __syncthreads();
  const int col0 = wg * kCols + grp * 4;
#pragma unroll
  for (int hg = 0; hg < kG; ++hg) {
    const int h = g * kHalf + hg * 16 + li;
    const float lf = sh.l_fin[h];
    if (a.n_splits == 1) {
      const float inv = lf > 0.f ? 1.f / lf : 0.f;
      const int64_t obase = (static_cast<int64_t>(j) * a.n_heads + h) * kMlaDl + col0;
      if (a.out_dtype == DS_BF16) {
        uint16_t* out = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          uint2 pk;
          pk.x = f32_to_bf16_bits(o[cb][hg][0] * inv) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(o[cb][hg][1] * inv)) << 16);
          pk.y = f32_to_bf16_bits(o[cb][hg][2] * inv) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(o[cb][hg][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(out + cb * 16) = pk;
        }
      } else {
        float* out = static_cast<float*>(a.out) + obase;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          *reinterpret_cast<float4*>(out + cb * 16) =
              make_float4(o[cb][hg][0] * inv, o[cb][hg][1] * inv, o[cb][hg][2] * inv,
                          o[cb][hg][3] * inv);
      }
    } else {
      uint16_t* po = mla_partial_o(a, j, split, h) + col0;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
        mla_store_bf16x4(po + cb * 16, o[cb][hg][0], o[cb][hg][1], o[cb][hg][2], o[cb][hg][3]);
    }
  }
  if (lane < 16) {
    if (a.n_splits == 1) {
      if (a.lse)
        a.lse[static_cast<int64_t>(j) * a.n_heads + h_own] =
            l_run > 0.f ? (m_ref + log2f(l_run)) * kLn2 : -INFINITY;
    } else {
      float* pml = mla_partial_ml(a, j, split, h_own);
      pml[0] = m_ref;
      pml[1] = l_run;
    }
  }
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
// accumulators are only ever touched by MFMA).  A later tile whose maximum
// exceeds the reference by more than 2^kWideBail (weights up to 2^64 are
// exact in fp32/bf16 range terms) makes the workgroup start over with the
// exact maximum from a first pass over all its rows.
constexpr float kWideBail = 64.f;

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
__device__ __forceinline__ int wide_off(int r, int x) {
  const int hh = (x >> 4) & 1;
  return (x >> 5) * 1024 + hh * 512 + (r ^ (hh << 3)) * 16 + (x & 15);
}
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

// The global byte offset a lane gathers from for every DMA instruction of a
// tile: its row (empty slots, -1, read row 0: their logits are masked and
// their softmax weight is 0) and its half.  32-bit: the latent KV must be
// smaller than 4 GiB.
__device__ __forceinline__ uint32_t wide_gather_base(int32_t row, int l) {
  row = row < 0 ? 0 : row;
  return static_cast<uint32_t>(row) * kMlaRowBytes + static_cast<uint32_t>((l >> 5) << 4);
}
// One DMA wave-instruction: block m of the tile at LDS address lds (the
// block's start: lane l lands at lds + 16l) from bytes [32m, 32m+32) of the
// lane's row.
__device__ __forceinline__ void wide_gather_issue(const uint8_t* kv, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(kv), "s"(lds)
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

template <bool kTrV, int kNW, bool kLag>
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
  for (int32_t i = n_valid + tid; i < (n_tiles + 1) * kPipeTile; i += kThreads) sh.sidx[i] = -1;
  if (tid < kNW) sh.bail[tid] = 0;
  const float scale2 = a.sm_scale * kLog2e;
  const uint8_t* kv = static_cast<const uint8_t*>(a.kv);
  const uint32_t lds_bufs = static_cast<uint32_t>(
      (size_t)((__attribute__((address_space(3))) uint8_t*)g_mla_bufs));
  // wave w issues blocks w, w + kNW, ...: slot i is block kNW*i + wave
  auto slot_lds = [&](int b, int i) {
    return lds_bufs + static_cast<uint32_t>(b * kPipeTileBytes + (kNW * i + wave) * 1024);
  };
  auto slot_off = [&](uint32_t base, int i) { return base + static_cast<uint32_t>(32 * (kNW * i + wave)); };
  auto row_of = [&](int t0) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return wide_gather_base(sh.sidx[t0 + wide_gather_slot(ln)], ln);
  };
  // all of this wave's slots of the tile with rows sidx[t0..] into buffer b
  auto issue_tile = [&](int b, int t0) {
    const uint32_t base = row_of(t0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) wide_gather_issue(kv, slot_lds(b, i), slot_off(base, i));
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
  // tile (rows sidx[t0g..], into gbuf) spread over the k-steps
  auto qk = [&](const uint8_t* tile, f32x4 (&st)[2][2], bool gather, int t0g, int gb) {
    // the gather's row is read first, so that waiting for it does not wait
    // for the K fragment reads behind it
    const uint32_t gbase = gather ? row_of(t0g) : 0u;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int koff = wide_koff(ln);
    auto kfrag = [&](int kb, int ks) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(tile + koff + kb * 256 + ks * 2048));
    };
    f32x4 su[2][2];
    // K fragments are read kAhead k-steps before their products; the
    // scheduling barriers keep the compiler from sinking the reads next to
    // their use (one wave per SIMD: nothing else hides the LDS latency)
    constexpr int kAhead = 2;
    // k-steps over which the gather slots are spread: the lagged schedule
    // gathers only one tile ahead, so its slots go out in the first half
    constexpr int kSpread = kLag ? kMlaKSteps / 2 : kMlaKSteps;
    bf16x8 kf[kAhead + 1][2];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) {
      kf[s][0] = kfrag(0, s);
      kf[s][1] = kfrag(1, s);
    }
#pragma unroll
    for (int ks = 0; ks < kMlaKSteps; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      if (ks + kAhead < kMlaKSteps) {
        kf[(ks + kAhead) % (kAhead + 1)][0] = kfrag(0, ks + kAhead);
        kf[(ks + kAhead) % (kAhead + 1)][1] = kfrag(1, ks + kAhead);
      }
      const bf16x8 k0 = kf[ks % (kAhead + 1)][0], k1 = kf[ks % (kAhead + 1)][1];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bf16x8 qv = ks < kQReg ? qf[hb][ks < kQReg ? ks : 0]
                                     : __builtin_bit_cast(bf16x8, sh.qrope[ks - kQReg][grp][h0 + 16 * hb]);
        // even and odd k-steps accumulate separately: 8 independent chains
        f32x4 (&acc)[2][2] = (ks & 1) ? su : st;
        if (ks < 2) {
          acc[0][hb] = mla_qk_first(k0, qv);
          acc[1][hb] = mla_qk_first(k1, qv);
        } else {
          mla_qk_acc(acc[0][hb], k0, qv);
          mla_qk_acc(acc[1][hb], k1, qv);
        }
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i * kSpread / kPer == ks && gather) wide_gather_issue(kv, slot_lds(gb, i), slot_off(gbase, i));
      }
    }
    mla_qk_settle(st[0][0], st[0][1], st[1][0], st[1][1]);
    mla_qk_settle(su[0][0], su[0][1], su[1][0], su[1][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) st[kb][hb] += su[kb][hb];
  };
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
  //   pv_c: issue the PV products of the previous tile (V in vtile, P^T in
  //         parity buffer pb_rd); sm_c: run the softmax of st and write its
  //         P^T to parity buffer pb_wr.  Softmax without PV is the first
  //         tile, which also sets the reference maximum.
  auto phase_b = [&](auto pv_c, auto sm_c, const uint8_t* vtile, int pb_rd, int pb_wr,
                     f32x4 (&st)[2][2], bool& beyond) __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_c)::value;
    constexpr bool kSM = decltype(sm_c)::value;
    constexpr bool kFirst = !kPV;
    constexpr int kCBL = kCB < 8 ? kCB : 8;   // column blocks whose V fragments are held
    constexpr int kUnits = kCB * kHG;         // PV products per tile and wave
    static_assert(kUnits == 64, "64 PV products per tile and wave");
    static_assert(kCB == kCBL, "the lagged schedule holds every V fragment of the wave");
    float mx[2], nm[2], psum[2] = {0.f, 0.f};
    bf16x8 pvb[2];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int li_t = ln & 15, grp_t = ln >> 4;
    const int voff = wide_voff(ln, wave * kCols);
    bf16x8 vf[kCBL];
    bf16x8 pf[2];
    auto load_p = [&](int hg) {
      return __builtin_bit_cast(bf16x8, sh.p[pb_rd][grp_t][hg * 16 + li_t]);
    };
    if constexpr (kPV) {
#pragma unroll
      for (int c = 0; c < kCBL; ++c) {
        if constexpr (kTrV) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vtile + voff + c * 1024));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vtile + voff + 256 + c * 1024));
          vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          const int x = (wave * kCols + c * 16 + li_t) * 2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vf[c][i] = *reinterpret_cast<const __bf16*>(vtile + wide_off(4 * grp_t + i, x));
            vf[c][4 + i] = *reinterpret_cast<const __bf16*>(vtile + wide_off(16 + 4 * grp_t + i, x));
          }
        }
      }
      pf[0] = load_p(0);
    }
    // softmax pieces; u is a compile-time constant once the unit loop is
    // unrolled.  Values: st[kb][hb][i] is key 16kb + 4grp + i of head
    // h0 + 16hb; v = 8hb + 4kb + i.
    auto micro = [&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < 2) {                       // raw maximum of head block u
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
        beyond = (mx[0] > m_ref[0] + kWideBail) || (mx[1] > m_ref[1] + kWideBail);
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
          l_run[hb] += __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
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
        // the next head group's P^T fragment, read one group ahead
        if constexpr (c == 0 && hg + 1 < kHG) pf[(hg + 1) & 1] = load_p(hg + 1);
        o[c][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c], pf[hg & 1], o[c][hg], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (;;) {
    if (exact) {
      // ---- first pass: exact maximum of every head over all rows (tiles
      //      gathered one at a time into buffer 0)
      m_ref[0] = m_ref[1] = -INFINITY;
      for (int32_t t = 0; t < n_tiles; ++t) {
        __syncthreads();   // buffer 0 free
        issue_tile(0, t * kPipeTile);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        const int32_t my_row = lane < kPipeTile ? sh.sidx[t * kPipeTile + lane] : -1;
        const uint64_t valid = __ballot(my_row >= 0);
        f32x4 st[2][2];
        qk(g_mla_bufs, st, false, 0, 0);
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
      auto qk_tile = [&](int32_t t, int b, f32x4 (&st)[2][2]) __attribute__((always_inline)) {
        const uint8_t* tile = g_mla_bufs + b * kPipeTileBytes;
        // the gather of tile t+1 is issued unconditionally (after the last
        // tile it reads padding rows into a free buffer), so the k-step loop
        // has no branch; the epilogue waits for it before reusing the buffers
        qk(tile, st, true, (t + 1) * kPipeTile, b == 2 ? 0 : b + 1);
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
        qk_tile(0, 0, st);
        bool beyond = false;
        phase_b(no, yes, g_mla_bufs, 0, 0, st, beyond);
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
        qk_tile(t, b, st);
        bool beyond = false;
        phase_b(yes, yes, g_mla_bufs + (b == 0 ? 2 : b - 1) * kPipeTileBytes,
                (t - 1) & 1, t & 1, st, beyond);
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
          phase_b(yes, no, g_mla_bufs + bl * kPipeTileBytes, (n_tiles - 1) & 1, 0, st, beyond);
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
      int lr = lane;
      asm volatile("" : "+v"(lr));   // recomputed per tile, not kept (and spilled)
      const int32_t my_row = lr < kPipeTile ? sh.sidx[t * kPipeTile + lr] : -1;
      const uint64_t valid = __ballot(my_row >= 0);
      // ---- QK, with the gather of tile t+2 into the buffer of tile t-1
      f32x4 st[2][2];
      qk(tile, st, t + 2 < n_tiles, (t + 2) * kPipeTile, b == 0 ? 2 : b - 1);
      // ---- softmax weights relative to the fixed reference
      float mx[2];
      logits(st, valid, mx);
      bool beyond = false;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (t == 0 && !exact) m_ref[hb] = mx[hb];
        beyond |= mx[hb] > m_ref[hb] + kWideBail;
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
          if constexpr (kTrV) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(tile + voff + cb * 1024));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(tile + voff + 256 + cb * 1024));
            vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            const int x = (wave * kCols + cb * 16 + li) * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              vf[c][i] = *reinterpret_cast<const __bf16*>(tile + wide_off(4 * grp + i, x));
              vf[c][4 + i] = *reinterpret_cast<const __bf16*>(tile + wide_off(16 + 4 * grp + i, x));
            }
          }
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
// Value fragments are read with the LDS transpose instruction unless
// DS32CP_MLA_SCALAR_V=1 selects the element-wise reads (same results; used
// to cross-check the transpose layout).
static bool mla_lag() {
  const char* e = getenv("DS32CP_MLA_LAG");
  return !(e && e[0] == '0');
}
static bool mla_transpose_reads() {
  const char* e = getenv("DS32CP_MLA_SCALAR_V");
  return !(e && e[0] == '1');
}

// fp8 rows -> bf16 rows of code * scale (round to nearest even), 16 codes
// per thread: one 16-byte load, two 16-byte stores.
__global__ void __launch_bounds__(256)
widen_fp8_rows_kernel(const uint8_t* codes, const float* scale, int64_t rows, uint16_t* out) {
  constexpr int kPer = kMlaD / 16;   // 36 pieces of 16 codes per row
  const int64_t piece = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (piece >= rows * kPer) return;
  const int64_t r = piece / kPer;
  const float sc = scale[r / kFp8BlockRows];
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

ds_status launch_widen_fp8_rows(const void* codes, const float* scale, int64_t rows, void* out,
                                hipStream_t s) {
  if (rows <= 0) return DS_OK;
  const int64_t pieces = rows * (kMlaD / 16);
  widen_fp8_rows_kernel<<<static_cast<unsigned>(ceil_div(pieces, 256)), 256, 0, s>>>(
      static_cast<const uint8_t*>(codes), scale, rows, static_cast<uint16_t*>(out));
  return check_launch("sparse_mla (fp8 rows to bf16)");
}

int32_t mla_decode_splits(int32_t n_q, int32_t topk) {
  // enough workgroups to cover the 256 CUs; at least 4 tiles per split
  const int32_t tiles = static_cast<int32_t>(ceil_div(topk, kMlaTile));
  int32_t want = static_cast<int32_t>(ceil_div(256, n_q > 0 ? n_q : 1));
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
  const bool tr = mla_transpose_reads();
  // the wide kernel addresses rows with 32-bit offsets
  const bool wide = static_cast<uint64_t>(a.kv_rows) * kMlaRowBytes < (1ull << 32);
  if (a.kv_dtype == DS_BF16) {
    if (!wide) switch (a.n_heads) {
      case 32:
        if (tr) mla_bf16_pipelined_kernel<true, 1><<<blocks, kWave * 2, 0, s>>>(a, per_split);
        else mla_bf16_pipelined_kernel<false, 1><<<blocks, kWave * 2, 0, s>>>(a, per_split);
        break;
      case 64:
        if (tr) mla_bf16_pipelined_kernel<true, 2><<<blocks, kWave * 4, 0, s>>>(a, per_split);
        else mla_bf16_pipelined_kernel<false, 2><<<blocks, kWave * 4, 0, s>>>(a, per_split);
        break;
      default:
        if (tr) mla_bf16_pipelined_kernel<true, 4><<<blocks, kWave * 8, 0, s>>>(a, per_split);
        else mla_bf16_pipelined_kernel<false, 4><<<blocks, kWave * 8, 0, s>>>(a, per_split);
    }
    else switch (a.n_heads) {
      case 32:
        if (tr) mla_bf16_wide_kernel<true, 1, false><<<blocks, kWave * 1, 0, s>>>(a, per_split);
        else mla_bf16_wide_kernel<false, 1, false><<<blocks, kWave * 1, 0, s>>>(a, per_split);
        break;
      case 64:
        if (tr) mla_bf16_wide_kernel<true, 2, false><<<blocks, kWave * 2, 0, s>>>(a, per_split);
        else mla_bf16_wide_kernel<false, 2, false><<<blocks, kWave * 2, 0, s>>>(a, per_split);
        break;
      default:
        if (mla_lag()) {
          if (tr) mla_bf16_wide_kernel<true, 4, true><<<blocks, kWave * 4, 0, s>>>(a, per_split);
          else mla_bf16_wide_kernel<false, 4, true><<<blocks, kWave * 4, 0, s>>>(a, per_split);
        } else {
          if (tr) mla_bf16_wide_kernel<true, 4, false><<<blocks, kWave * 4, 0, s>>>(a, per_split);
          else mla_bf16_wide_kernel<false, 4, false><<<blocks, kWave * 4, 0, s>>>(a, per_split);
        }
    }
    ds_status st = check_launch("sparse_mla");
    if (st != DS_OK || a.n_splits == 1) return st;
    dim3 cgrid(a.n_q, a.n_heads / kMlaCombineHeads);
    mla_combine_kernel<<<cgrid, 256, 0, s>>>(a);
    return check_launch("sparse_mla combine");
  }
  const int threads = kWave * (a.n_heads / (16 * kMlaGroups));
  if (a.kv_dtype == DS_FP8_E4M3FN) {
    if (tr) mla_mfma_kernel<true, true, kMlaGroups><<<blocks, threads, 0, s>>>(a, per_split);
    else mla_mfma_kernel<true, false, kMlaGroups><<<blocks, threads, 0, s>>>(a, per_split);
  } else {
    if (tr) mla_mfma_kernel<false, true, kMlaGroups><<<blocks, threads, 0, s>>>(a, per_split);
    else mla_mfma_kernel<false, false, kMlaGroups><<<blocks, threads, 0, s>>>(a, per_split);
  }
  ds_status st = check_launch("sparse_mla");
  if (st != DS_OK || a.n_splits == 1) return st;
  dim3 cgrid(a.n_q, a.n_heads / kMlaCombineHeads);
  mla_combine_kernel<<<cgrid, 256, 0, s>>>(a);
  return check_launch("sparse_mla combine");
}

}  // namespace ds32cp
