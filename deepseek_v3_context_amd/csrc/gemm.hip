// The dense projections on either side of the path, as one batched GEMM.
//
// Sources: "Model Parallel Strategy Analysis", step 3.1 (MLA's projection
// structure: q_down / q_up / kv_down / kv_up (K and V) / o_proj);
// "[RFC]: Parallel strategy for Deepseek v3.2 like models", "Problem with
// tp" (the indexer's wq_b and w_k projections, which every rank would
// otherwise run on every token).  With the latent (absorbed) attention the
// up-projection of K folds into the queries (q_latent = q_nope . W_UK per
// head) and that of V into the output (o = O_latent . W_UV per head); both
// are batched over the heads.
//
//   C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]      (fp32 accumulation)
//
// A is M x K and B is N x K, both K-contiguous (weights stored as
// [out, in]), C is M x N; every operand has its own row and batch stride,
// so a per-head slice of a wider row (q_nope inside the q row, the latent
// part of the 576-wide MLA query) is addressed in place.
//
// Kernel: 8 waves per workgroup (two per SIMD), a BM x BN output tile, K in
// steps of 64.  Each step's A and B tiles (rows of 128 bytes) are copied
// into LDS by direct global->LDS loads into a ring of NS stages (two for
// 256 x 256 tiles, which is what LDS holds; three for 256 x 128), so that
// the copies of the next steps run under this step's products.  Within a tile row the
// eight 16-byte chunks are stored XOR-permuted by bits 2..3 of the row, so
// that the sixteen rows a 16-lane group reads for one MFMA fragment land in
// sixteen distinct 16-byte bank slots.  Products: v_mfma_f32_32x32x16_bf16,
// each wave a (BM/WM) x (BN/WN) sub-tile held in accumulator registers.
// The output tile goes out through LDS, 64 rows at a time, as 16-byte pieces
// of whole rows.  Split-K (few output tiles, long K): each split writes its
// fp32 partial tile to the workspace and a second kernel sums the splits in
// order.
#include "common.h"

namespace ds32cp {

namespace {

constexpr int kGemmBK = 64;                 // K per step (128 bytes of a row)
constexpr int kGemmThreads = 512;           // 8 waves

// LDS byte offset of 16-byte chunk c of tile row r (rows of RB bytes: 64
// or 128).  The XOR by bits 2..3 of the row puts the 16 rows that a 16-lane
// group reads for one fragment in 16 distinct 16-byte bank slots.
template <int RB>
__device__ __forceinline__ int gemm_lds_off(int r, int c) {
  return r * RB + ((c ^ ((r >> 2) & 3)) << 4);
}

// One direct global->LDS copy of 16 bytes per lane: lane l lands at
// lds + 16 l (lds: the instruction's block start, the same for the wave).
__device__ __forceinline__ void gemm_dma(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      (size_t)((__attribute__((address_space(3))) const uint8_t*)p));
}

}  // namespace

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding (expcnt and lgkmcnt left unconstrained)
constexpr int gemm_vmcnt(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

template <int BM, int BN, int WM, int WN, int NS, int BK>
__global__ void __launch_bounds__(kGemmThreads)
gemm_nt_kernel(GemmArgs g, int32_t tiles_m, int32_t tiles_n, int32_t k_per_split) {
  static_assert(WM * WN == kGemmThreads / kWave, "eight waves");
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  constexpr int ROWB = BK * 2;                    // bytes of a tile row
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int WTM = BM / WM, WTN = BN / WN;     // wave sub-tile
  constexpr int FM = WTM / 32, FN = WTN / 32;     // 32 x 32 blocks per wave
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_INST = A_BYTES / (kGemmThreads * 16);   // copies per thread and step
  constexpr int B_INST = B_BYTES / (kGemmThreads * 16);
  constexpr int PER = A_INST + B_INST;                    // vector-memory ops per step
  static_assert(A_INST >= 1 && B_INST >= 1, "a tile is at least one copy per thread");
  static_assert((NS - 2) * PER <= 63, "the wait count fits the counter");
  __shared__ __align__(16) uint8_t smem[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;

  // workgroup -> (batch, split, tile): consecutive logical ids run on one
  // XCD and walk the tiles in groups of kGroupM row blocks, the row block
  // varying fastest, so that the XCD's concurrent tiles (about 32) span a
  // few A row blocks and a few B column blocks, which its L2 then serves to
  // all of them (o_proj on 8192 tokens: 1905 -> 1790-1800 us against
  // N tiles varying fastest)
  int64_t id = (gridDim.x & 7u) == 0 ? xcd_contiguous_id(blockIdx.x, gridDim.x) : blockIdx.x;
  constexpr int32_t kGroupM = 8;
  const int64_t per_bs = static_cast<int64_t>(tiles_m) * tiles_n;
  const int32_t t_in = static_cast<int32_t>(id % per_bs);
  id /= per_bs;
  const int32_t first_m = (t_in / (kGroupM * tiles_n)) * kGroupM;
  const int32_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int32_t in_group = t_in - first_m * tiles_n;
  const int32_t tm = first_m + in_group % gm;
  const int32_t tn = in_group / gm;
  const int32_t split = static_cast<int32_t>(id % g.splits);
  const int32_t b = static_cast<int32_t>(id / g.splits);
  const int32_t m0 = tm * BM, n0 = tn * BN;
  const int32_t k_begin = split * k_per_split;
  const int32_t k_steps = (min(g.K, k_begin + k_per_split) - k_begin) / BK;

  const uint8_t* A = static_cast<const uint8_t*>(g.A) + (b * g.strideA + k_begin) * 2;
  const uint8_t* B = static_cast<const uint8_t*>(g.B) + (b * g.strideB + k_begin) * 2;
  // per-lane source of each copy: LDS chunk q = i*512 + tid holds row
  // q/CPR, stored chunk q%CPR, i.e. global chunk (q%CPR) ^ ((row >> 2) & 3);
  // rows past M (N) read the last valid row, whose products are never stored
  const uint8_t* a_src[A_INST];
  const uint8_t* b_src[B_INST];
#pragma unroll
  for (int i = 0; i < A_INST; ++i) {
    const int q = i * kGemmThreads + tid, r = q / CPR;
    const int gc = (q % CPR) ^ ((r >> 2) & 3);
    const int64_t row = min(m0 + r, g.M - 1);
    a_src[i] = A + row * g.lda * 2 + gc * 16;
  }
#pragma unroll
  for (int i = 0; i < B_INST; ++i) {
    const int q = i * kGemmThreads + tid, r = q / CPR;
    const int gc = (q % CPR) ^ ((r >> 2) & 3);
    const int64_t row = min(n0 + r, g.N - 1);
    b_src[i] = B + row * g.ldb * 2 + gc * 16;
  }
  const uint32_t s0 = lds_addr(smem);
  auto issue = [&](int stage, int kt) {
    const uint32_t base = s0 + stage * STAGE;
    const int64_t koff = static_cast<int64_t>(kt) * BK * 2;
#pragma unroll
    for (int i = 0; i < A_INST; ++i)
      gemm_dma(a_src[i] + koff, base + (i * kGemmThreads + wave * kWave) * 16);
#pragma unroll
    for (int i = 0; i < B_INST; ++i)
      gemm_dma(b_src[i] + koff, base + A_BYTES + (i * kGemmThreads + wave * kWave) * 16);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment offsets: lane l reads row (l % 32) of a 32-row block and
  // chunk 2 kk + l / 32 for k-substep kk
  const int fr = lane & 31, fh = lane >> 5;
  // NS-stage ring: the copies of step kt + NS - 1 go out right after the
  // barrier of step kt, into the stage that step kt - 1 read
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < k_steps) issue(p, p);
  for (int kt = 0; kt < k_steps; ++kt) {
    const int st = kt % NS;
    // this wave's copies of step kt landed: the younger steps' copies
    // (up to NS - 2 of them, fewer near the end) may stay in flight
    const int younger = min(NS - 2, k_steps - 1 - kt);
    if (NS >= 4 && younger >= 2) __builtin_amdgcn_s_waitcnt(gemm_vmcnt(2 * PER));
    else if (NS >= 3 && younger >= 1) __builtin_amdgcn_s_waitcnt(gemm_vmcnt(PER));
    else __builtin_amdgcn_s_waitcnt(gemm_vmcnt(0));
    __syncthreads();                 // everyone's; and step kt-1's reads are done
    if (kt + NS - 1 < k_steps) issue((kt + NS - 1) % NS, kt + NS - 1);
    const uint8_t* sa = smem + st * STAGE;
    const uint8_t* sb = sa + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + fr;
        af[i] = *reinterpret_cast<const bf16x8*>(sa + gemm_lds_off<ROWB>(r, 2 * kk + fh));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 32 + fr;
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + gemm_lds_off<ROWB>(r, 2 * kk + fh));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane l holds column l % 32 of each block, rows
  // 8 (e / 4) + 4 (l / 32) + e % 4
  if (g.splits > 1) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int32_t col = n0 + wn * WTN + j * 32 + fr;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
          if (row >= g.M) continue;
          float* p = static_cast<float*>(g.ws) +
                     ((static_cast<int64_t>(split) * g.batch + b) * g.M + row) * g.N + col;
          *p = acc[i][j][e];
        }
      }
    return;
  }
  // The output goes out through LDS (free after the last step) 64 rows at
  // a time, so that the global stores are 16-byte pieces of whole rows; a
  // lane's own elements are single values of 32 different rows.
  auto write_out = [&](auto esz) __attribute__((always_inline)) {
    constexpr int E = decltype(esz)::value;      // bytes per element
    constexpr int RB = 64;                       // rows per block
    constexpr int RS = BN * E + 16;              // padded LDS row
    static_assert(RB * RS <= NS * STAGE, "a row block fits in the stages");
    constexpr int PIECES = BN * E / 16;          // 16-byte pieces per row
    uint8_t* C = static_cast<uint8_t*>(g.C) + (static_cast<int64_t>(b) * g.strideC + n0) * E;
    const bool vec = ((reinterpret_cast<uintptr_t>(C) | static_cast<uintptr_t>(g.ldc * E)) & 15u) == 0;
#pragma unroll
    for (int rb = 0; rb < BM / RB; ++rb) {
      __syncthreads();   // the stages (and the previous block) are free
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if ((wm * WTM + i * 32) / RB != rb) continue;   // uniform per wave
        const int r0 = wm * WTM + i * 32 - rb * RB;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = wn * WTN + j * 32 + fr;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = r0 + 8 * (e >> 2) + 4 * fh + (e & 3);
            if constexpr (E == 2) {
              *reinterpret_cast<uint16_t*>(smem + r * RS + col * 2) = f32_to_bf16_bits(acc[i][j][e]);
            } else {
              *reinterpret_cast<float*>(smem + r * RS + col * 4) = acc[i][j][e];
            }
          }
        }
      }
      __syncthreads();
      constexpr int TOTAL = RB * PIECES;
#pragma unroll
      for (int q0 = 0; q0 < TOTAL; q0 += kGemmThreads) {
        const int q = q0 + tid;
        const int r = q / PIECES, c = q - (q / PIECES) * PIECES;
        const int32_t row = m0 + rb * RB + r;
        if (q < TOTAL && row < g.M) {
          const uint4 v = *reinterpret_cast<const uint4*>(smem + r * RS + c * 16);
          uint8_t* dst = C + static_cast<int64_t>(row) * g.ldc * E + c * 16;
          if (vec) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              if constexpr (E == 2) {
                reinterpret_cast<uint16_t*>(dst)[2 * k] = static_cast<uint16_t>(w[k] & 0xffffu);
                reinterpret_cast<uint16_t*>(dst)[2 * k + 1] = static_cast<uint16_t>(w[k] >> 16);
              } else {
                reinterpret_cast<uint32_t*>(dst)[k] = w[k];
              }
            }
          }
        }
      }
    }
  };
  if (g.c_dtype == DS_BF16) write_out(std::integral_constant<int, 2>{});
  else write_out(std::integral_constant<int, 4>{});
}

// Sum of the split partials, in split order, then the output conversion.
__global__ void __launch_bounds__(256)
gemm_splitk_reduce_kernel(GemmArgs g) {
  const int64_t total = static_cast<int64_t>(g.batch) * g.M * g.N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const float* ws = static_cast<const float*>(g.ws);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += stride) {
    float s = 0.f;
    for (int32_t k = 0; k < g.splits; ++k) s += ws[k * total + e];
    const int64_t n = e % g.N, t = e / g.N, m = t % g.M, b = t / g.M;
    const int64_t off = b * g.strideC + m * g.ldc + n;
    if (g.c_dtype == DS_BF16) static_cast<uint16_t*>(g.C)[off] = f32_to_bf16_bits(s);
    else static_cast<float*>(g.C)[off] = s;
  }
}

// Output tile width: 256 when N allows it, except when 256-wide tiles
// would leave CUs idle (and so need split-K) while 128-wide ones cover
// every CU without it (q_down on 8192 tokens, N = 1536: 192 wide tiles and
// a 3-way split with its sum, 281 us, against 384 narrow tiles, 235 us).
static int32_t gemm_tile_n(int32_t M, int32_t N, int32_t batch) {
  if (N % 256 != 0) return 128;
  const int64_t rows = ceil_div(M, 256) * static_cast<int64_t>(batch);
  const int64_t cus = device_cu_count();
  return rows * (N / 256) < cus && rows * (N / 128) >= cus ? 128 : 256;
}

int32_t gemm_splits(int32_t M, int32_t N, int32_t K, int32_t batch) {
  const int64_t bn = gemm_tile_n(M, N, batch);
  const int64_t tiles = ceil_div(M, 256) * (N / bn) * static_cast<int64_t>(batch);
  const int64_t cus = device_cu_count();
  const int64_t steps = K / kGemmBK;
  if (tiles >= cus || steps < 16) return 1;
  int64_t s = ceil_div(2 * cus, tiles);
  s = s < steps / 8 ? s : steps / 8;        // at least 8 steps per split
  s = s < 16 ? s : 16;
  return static_cast<int32_t>(s > 1 ? s : 1);
}

ds_status launch_gemm(GemmArgs g, hipStream_t s) {
  if (g.M == 0 || g.N == 0 || g.batch == 0) return DS_OK;
  const int32_t k_steps = g.K / kGemmBK;
  const int32_t per = static_cast<int32_t>(ceil_div(k_steps, g.splits)) * kGemmBK;
  const int32_t tiles_m = static_cast<int32_t>(ceil_div(g.M, 256));
  if (gemm_tile_n(g.M, g.N, g.batch) == 256) {
    const int32_t tiles_n = g.N / 256;
    const int64_t blocks = static_cast<int64_t>(tiles_m) * tiles_n * g.splits * g.batch;
    gemm_nt_kernel<256, 256, 2, 4, 2, 64><<<static_cast<unsigned>(blocks), kGemmThreads, 0, s>>>(
        g, tiles_m, tiles_n, per);
  } else {
    const int32_t tiles_n = g.N / 128;
    const int64_t blocks = static_cast<int64_t>(tiles_m) * tiles_n * g.splits * g.batch;
    gemm_nt_kernel<256, 128, 4, 2, 3, 64><<<static_cast<unsigned>(blocks), kGemmThreads, 0, s>>>(
        g, tiles_m, tiles_n, per);
  }
  ds_status st = check_launch("gemm_bf16_nt");
  if (st != DS_OK || g.splits == 1) return st;
  const int64_t total = static_cast<int64_t>(g.batch) * g.M * g.N;
  const int64_t want = ceil_div(total, 256);
  gemm_splitk_reduce_kernel<<<static_cast<unsigned>(want < 16384 ? want : 16384), 256, 0, s>>>(g);
  return check_launch("gemm_bf16_nt (split-K sum)");
}

}  // namespace ds32cp
