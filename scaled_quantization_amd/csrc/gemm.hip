// gemm.hip -- scaled FP8 x FP8 GEMM with FP32 accumulation and BF16 output.
//
// "FP8 training: what it is and how it works", Step 3: the multiplication
// reads FP8 inputs and keeps its running sum in a wider format; partial sums
// are promoted to FP32 every 128 elements.  "FP8 Training & Inference",
// Per-Tensor Scaling: the scales are factored out of the matmul and the
// output is rescaled.  Trade-offs: 1 x 128 activation tiles and 128 x 128
// weight blocks each carry their own scale.
//
//   y[m, n] = bf16_rne( sum_k dec(a[m, k]) dec(b[n, k]) * sa * sb )        per tensor
//   y[m, n] = bf16_rne( sum_g P_g[m, n] * sa[m, g] * sb[n/128, g] )      per group,
//             P_g = FP32 MFMA sum over the 128 k of block g
//
// Kernel (gfx950): a 256-thread workgroup owns a 128 x 128 tile of y; each of
// its four waves owns 64 x 64 as 2 x 2 tiles of v_mfma_f32_32x32x64_f8f6f4
// (the format of each operand is selected by the instruction's cbsz / blgp
// fields: 0 = E4M3, 1 = E5M2).  K advances 128 bytes at a time; A and B tiles
// (128 rows x 128 bytes each) are staged in LDS, double-buffered, with the
// 16-byte chunk c of row r stored at chunk c ^ (r & 7) so the 16-byte LDS
// reads of eight consecutive rows hit distinct banks.  Global loads for the
// next K step are issued before the MFMAs of the current one.
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "common.hpp"

namespace fp8dp {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));

// Widens the 32 FP8 codes of an MFMA fragment into four groups of 8 FP16
// values (exact: every E4M3 and E5M2 value is an FP16 value); group j holds
// bytes 8j .. 8j+7 in order.
template <int F>
__device__ __forceinline__ void widen_fp8(const v8i_t& x, v8h_t out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v2h_t p0, p1, p2, p3;
    if constexpr (F == 0) {
      p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[2 * j], 1.0f, false);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[2 * j], 1.0f, true);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[2 * j + 1], 1.0f, false);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[2 * j + 1], 1.0f, true);
    } else {
      p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(x[2 * j], 1.0f, false);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(x[2 * j], 1.0f, true);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(x[2 * j + 1], 1.0f, false);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(x[2 * j + 1], 1.0f, true);
    }
    out[j] = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                     __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                     5, 6, 7);
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kGemmThreads = 256;

__device__ __forceinline__ int swz(int r, int chunk) { return r * kBK + ((chunk ^ (r & 7)) << 4); }

// blockIdx -> output tile.  Workgroups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8); renumbering so that each XCD receives a
// contiguous run of tiles keeps tiles that share A rows in one XCD's L2.
__device__ __forceinline__ int tile_of_block(int b, int ntiles) {
  const int per = ntiles / 8;
  if (per * 8 != ntiles) return b;
  return (b % 8) * per + b / 8;
}

template <int FA, int FB, int MODE, bool EXACT>
__global__ __launch_bounds__(kGemmThreads, 2) void k_gemm(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ B, int M,
                                                          int N, int K,
                                                          const float* __restrict__ sa,
                                                          const float* __restrict__ sb,
                                                          uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBM * kBK];
  __shared__ float lds_sa[2][kBM];

  const int tiles_n = N / kBN;
  const int ntiles = (M / kBM) * tiles_n;
  const int tile = tile_of_block(blockIdx.x, ntiles);
  const int m0 = (tile / tiles_n) * kBM;
  const int n0 = (tile % tiles_n) * kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * 64;   // wave's row offset in the tile
  const int wn = (wave & 1) * 64;    // wave's column offset
  const int kgroups = K / kBK;

  // Global -> register staging: thread t moves chunks t + 256 i (i = 0..3) of
  // each 128 x 128-byte tile: row (t + 256 i) / 8, 16-byte chunk t % 8.
  const int srow = tid >> 3, sch = tid & 7;
  const uint8_t* gA = A + (size_t)(m0 + srow) * K + sch * 16;
  const uint8_t* gB = B + (size_t)(n0 + srow) * K + sch * 16;
  const size_t gstep = (size_t)32 * K;   // 256 threads / 8 chunks = 32 rows apart
  u32x4_t ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  float rsa = 0.0f;
#define FP8DP_GLOAD(kt)                                                                  \
  do {                                                                                   \
    const size_t k0 = (size_t)(kt) * kBK;                                                \
    ra0 = *reinterpret_cast<const u32x4_t*>(gA + k0);                                    \
    ra1 = *reinterpret_cast<const u32x4_t*>(gA + gstep + k0);                            \
    ra2 = *reinterpret_cast<const u32x4_t*>(gA + 2 * gstep + k0);                        \
    ra3 = *reinterpret_cast<const u32x4_t*>(gA + 3 * gstep + k0);                        \
    rb0 = *reinterpret_cast<const u32x4_t*>(gB + k0);                                    \
    rb1 = *reinterpret_cast<const u32x4_t*>(gB + gstep + k0);                            \
    rb2 = *reinterpret_cast<const u32x4_t*>(gB + 2 * gstep + k0);                        \
    rb3 = *reinterpret_cast<const u32x4_t*>(gB + 3 * gstep + k0);                        \
    if constexpr (MODE == FP8DP_PER_GROUP128) {                                          \
      if (tid < kBM) rsa = sa[(size_t)(m0 + tid) * kgroups + (kt)];                      \
    }                                                                                    \
  } while (0)
#define FP8DP_SSTORE(buf)                                                                \
  do {                                                                                   \
    *reinterpret_cast<u32x4_t*>(&lds[buf][0][swz(srow, sch)]) = ra0;                     \
    *reinterpret_cast<u32x4_t*>(&lds[buf][0][swz(srow + 32, sch)]) = ra1;                \
    *reinterpret_cast<u32x4_t*>(&lds[buf][0][swz(srow + 64, sch)]) = ra2;                \
    *reinterpret_cast<u32x4_t*>(&lds[buf][0][swz(srow + 96, sch)]) = ra3;                \
    *reinterpret_cast<u32x4_t*>(&lds[buf][1][swz(srow, sch)]) = rb0;                     \
    *reinterpret_cast<u32x4_t*>(&lds[buf][1][swz(srow + 32, sch)]) = rb1;                \
    *reinterpret_cast<u32x4_t*>(&lds[buf][1][swz(srow + 64, sch)]) = rb2;                \
    *reinterpret_cast<u32x4_t*>(&lds[buf][1][swz(srow + 96, sch)]) = rb3;                \
    if constexpr (MODE == FP8DP_PER_GROUP128) {                                          \
      if (tid < kBM) lds_sa[buf][tid] = rsa;                                             \
    }                                                                                    \
  } while (0)

  v16f_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  FP8DP_GLOAD(0);
  FP8DP_SSTORE(0);
  __syncthreads();

  const int frow = lane & 31;        // row of A / column of B this lane feeds
  const int fhalf = (lane >> 5) * 2; // which 32-byte half of each 64-wide K step

  for (int kt = 0; kt < kgroups; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < kgroups) FP8DP_GLOAD(kt + 1);

    v16f_t part[2][2];
    if constexpr (MODE == FP8DP_PER_GROUP128) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i_t fa[2], fb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra_row = wm + t * 32 + frow;
        const int rb_row = wn + t * 32 + frow;
        const int c0 = ks * 4 + fhalf;
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(&lds[buf][0][swz(ra_row, c0)]);
        const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(&lds[buf][0][swz(ra_row, c0 + 1)]);
        const u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(&lds[buf][1][swz(rb_row, c0)]);
        const u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(&lds[buf][1][swz(rb_row, c0 + 1)]);
        fa[t] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        fb[t] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      if constexpr (EXACT) {
        v8h_t ha[2][4], hb[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          widen_fp8<FA>(fa[t], ha[t]);
          widen_fp8<FB>(fb[t], hb[t]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if constexpr (MODE == FP8DP_PER_GROUP128)
                part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[i][q], hb[j][q], part[i][j],
                                                                    0, 0, 0);
              else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[i][q], hb[j][q], acc[i][j],
                                                                   0, 0, 0);
            }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (MODE == FP8DP_PER_GROUP128)
              part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  fa[i], fb[j], part[i][j], FA, FB, 0, 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  fa[i], fb[j], acc[i][j], FA, FB, 0, 0, 0, 0);
          }
      }
    }
    if constexpr (MODE == FP8DP_PER_GROUP128) {
      // promote the 128-wide partial sums with their scales
      const float sbv = sb[(size_t)(n0 / kBN) * kgroups + kt];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const float f = lds_sa[buf][row] * sbv;
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j][r] = __builtin_fmaf(part[i][j][r], f, acc[i][j][r]);
        }
    }
    if (kt + 1 < kgroups) FP8DP_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef FP8DP_GLOAD
#undef FP8DP_SSTORE

  float f = 1.0f;
  if constexpr (MODE == FP8DP_PER_TENSOR) f = sa[0] * sb[0];
  // Output layout of a 32 x 32 MFMA tile: lane holds column lane % 32, and
  // register r holds row 8 (r / 4) + 4 (lane / 32) + r % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = n0 + wn + j * 32 + (lane & 31);
        const float v = (MODE == FP8DP_PER_TENSOR) ? acc[i][j][r] * f : acc[i][j][r];
        Y[(size_t)row * N + col] = (uint16_t)bf16_rne_int(v);
      }
}

// ------------------------------------------------------------------ large tiles
// Per-tensor FP8 path for large problems.  A workgroup of WM x WN waves owns a
// BM x BN tile (256 x 192, 256 x 256 or 256 x 128 with 4 x 2 waves: 64 x 96,
// 64 x 128 or 64 x 64 per wave, as 32 x 32 MFMA tiles), two waves per SIMD so
// one wave's LDS reads overlap the other's MFMAs.  K advances 128 bytes per
// stage through two LDS stages: the copies of stage t+1 are issued before the
// MFMAs of stage t.  Global memory is copied straight into LDS with
// global_load_lds_dwordx4 (no register staging): one instruction moves 64
// lanes x 16 bytes = 8 rows of 128 bytes, lane i landing at byte 16 i; lane i
// therefore fetches global chunk (i % 8) ^ (i / 8) of row i / 8, which is the
// same XOR swizzle as the small-tile kernel (chunk c of row r at c ^ (r & 7)).
// The epilogue pairs adjacent output columns between neighbour lanes (one DPP
// swap) and stores BF16 pairs straight to Y.
// Measured alternatives (GPT-2 shape): 64-byte stages with a 4-5 deep ring,
// and fragment reads interleaved between MFMAs, were both slower on gfx950.
typedef __attribute__((address_space(3))) void lds_void_t;

template <int FA, int FB, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_gemm_big(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ B,
                                                              int M, int N, int K,
                                                              const float* __restrict__ sa,
                                                              const float* __restrict__ sb,
                                                              uint16_t* __restrict__ Y) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;     // 32 x 32 MFMA tiles per wave
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wave tiling");
  constexpr int STAGE = (BM + BN) * kBK;                  // bytes of one LDS stage
  constexpr int A_LOADS = BM / 8 / NW, B_LOADS = BN / 8 / NW;   // 1-KiB copies per wave
  static_assert(A_LOADS * 8 * NW == BM && B_LOADS * 8 * NW == BN, "copy split");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tiles_n = N / BN;
  const int ntiles = (M / BM) * tiles_n;
  const int tile = tile_of_block(blockIdx.x, ntiles);
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = (wave / WN) * (BM / WM);
  const int wc = (wave % WN) * (BN / WN);
  const int KT = K / kBK;

  // this lane's source within each 8-row copy: row lane / 8, chunk (lane % 8) ^ (lane / 8)
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  const uint8_t* gA = A + (size_t)(m0 + wave * 8 + lrow) * K + lchunk * 16;
  const uint8_t* gB = B + (size_t)(n0 + wave * 8 + lrow) * K + lchunk * 16;
  const size_t rstep = (size_t)(8 * NW) * K;              // the waves cover 8 NW rows per round

  auto issue = [&](int kt) {
    const size_t k0 = (size_t)kt * kBK;
    uint8_t* base = lds + (kt & 1) * STAGE;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      __builtin_amdgcn_global_load_lds(gA + i * rstep + k0,
                                       (lds_void_t*)(base + (i * 8 * NW + wave * 8) * kBK), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      __builtin_amdgcn_global_load_lds(
          gB + i * rstep + k0, (lds_void_t*)(base + BM * kBK + (i * 8 * NW + wave * 8) * kBK),
          16, 0, 0);
  };

  v16f_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int frow = lane & 31;
  const int fhalf = (lane >> 5) * 2;
  issue(0);
  for (int kt = 0; kt < KT; ++kt) {
    // This wave's copies of stage kt have landed; the barrier makes every
    // wave's copies visible, and shows every wave is done with stage kt-1,
    // whose slot the copies of stage kt+1 refill.  (A full __syncthreads()
    // would be equivalent here: nothing else is in flight.)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (kt + 1 < KT) issue(kt + 1);
    const uint8_t* sA = lds + (kt & 1) * STAGE;
    const uint8_t* sB = sA + BM * kBK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c0 = ks * 4 + fhalf;
      v8i_t fa[TM], fb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int r = wr + t * 32 + frow;
        const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(sA + swz(r, c0));
        const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(sA + swz(r, c0 + 1));
        fa[t] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wc + t * 32 + frow;
        const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(sB + swz(r, c0));
        const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(sB + swz(r, c0 + 1));
        fb[t] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], FA,
                                                                     FB, 0, 0, 0, 0);
    }
  }

  // epilogue: scale, round to BF16 and store pairs of adjacent columns.  In a
  // 32 x 32 MFMA tile the lane holds column lane % 32 and register r holds row
  // 8 (r / 4) + 4 (lane / 32) + r % 4; swapping one value with the neighbour
  // lane (DPP quad_perm 1,0,3,2) gives the even lane columns (c, c+1) of row
  // r and the odd lane the same columns of row r+1.
  const float f = sa[0] * sb[0];
  const bool odd = lane & 1;
  const int colp = (lane & 31) & ~1;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float v0 = acc[i][j][r] * f, v1 = acc[i][j][r + 1] * f;
        const float give = odd ? v0 : v1;
        const float got = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, give), 0xB1, 0xF, 0xF,
                                               false));
        const uint32_t packed = odd ? pack2_bf16_hw(got, v1) : pack2_bf16_hw(v0, got);
        const int row = m0 + wr + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + (odd ? 1 : 0);
        const int col = n0 + wc + j * 32 + colp;
        *reinterpret_cast<uint32_t*>(Y + (size_t)row * N + col) = packed;
      }
}

template <int FA, int FB, int BM, int BN>
static int launch_big(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                      const float* sa, const float* sb, uint16_t* y, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_big<FA, FB, BM, BN, 4, 2>), dim3((unsigned)((M / BM) * (N / BN))),
                     dim3(64 * 8), 0, stream, a, b, (int)M, (int)N, (int)K, sa, sb, y);
  return check_launch("fp8_gemm_scaled");
}

template <int FA, int FB, int MODE, bool EXACT>
static void launch_gemm_t(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                          const float* sa, const float* sb, uint16_t* y, hipStream_t stream) {
  const unsigned blocks = (unsigned)((M / kBM) * (N / kBN));
  hipLaunchKernelGGL((k_gemm<FA, FB, MODE, EXACT>), dim3(blocks), dim3(kGemmThreads), 0, stream,
                     a, b, (int)M, (int)N, (int)K, sa, sb, y);
}

template <int FA, int FB>
static int launch_gemm(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                       fp8dp_scale_mode mode, fp8dp_accum accum, const float* sa, const float* sb,
                       uint16_t* y, hipStream_t stream) {
  const bool exact = accum == FP8DP_ACCUM_EXACT;
  if (mode == FP8DP_PER_TENSOR && !exact && M % 256 == 0) {
    // the largest tile with at most one workgroup per compute unit at a time
    if (N % 192 == 0) return launch_big<FA, FB, 256, 192>(a, b, M, N, K, sa, sb, y, stream);
    if (N % 256 == 0) return launch_big<FA, FB, 256, 256>(a, b, M, N, K, sa, sb, y, stream);
    return launch_big<FA, FB, 256, 128>(a, b, M, N, K, sa, sb, y, stream);
  }
  if (mode == FP8DP_PER_TENSOR) {
    if (exact) launch_gemm_t<FA, FB, FP8DP_PER_TENSOR, true>(a, b, M, N, K, sa, sb, y, stream);
    else launch_gemm_t<FA, FB, FP8DP_PER_TENSOR, false>(a, b, M, N, K, sa, sb, y, stream);
  } else {
    if (exact) launch_gemm_t<FA, FB, FP8DP_PER_GROUP128, true>(a, b, M, N, K, sa, sb, y, stream);
    else launch_gemm_t<FA, FB, FP8DP_PER_GROUP128, false>(a, b, M, N, K, sa, sb, y, stream);
  }
  return check_launch("fp8_gemm_scaled");
}

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int fp8_gemm_scaled(const uint8_t* a, fp8dp_format fa, const uint8_t* b,
                               fp8dp_format fb, int64_t M, int64_t N, int64_t K,
                               fp8dp_scale_mode mode, fp8dp_accum accum,
                               const float* a_scale_inv, const float* b_scale_inv, uint16_t* y,
                               hipStream_t stream) {
  if (a == nullptr || b == nullptr || y == nullptr || a_scale_inv == nullptr ||
      b_scale_inv == nullptr) {
    set_error("fp8_gemm_scaled: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (M < kBM || N < kBN || K < kBK || M % kBM || N % kBN || K % kBK) {
    set_error("fp8_gemm_scaled: M, N, K must be positive multiples of 128 (got %lld, %lld, %lld)",
              (long long)M, (long long)N, (long long)K);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30 ||
      (M / kBM) * (N / kBN) > (int64_t)0x7FFFFFFF) {
    set_error("fp8_gemm_scaled: shape too large");
    return FP8DP_EINVAL;
  }
  if ((fa != FP8DP_E4M3 && fa != FP8DP_E5M2) || (fb != FP8DP_E4M3 && fb != FP8DP_E5M2) ||
      (mode != FP8DP_PER_TENSOR && mode != FP8DP_PER_GROUP128) ||
      (accum != FP8DP_ACCUM_MFMA_FP8 && accum != FP8DP_ACCUM_EXACT)) {
    set_error("fp8_gemm_scaled: unknown format, scale mode or accumulation mode");
    return FP8DP_EINVAL;
  }
  if (!aligned16(a) || !aligned16(b) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(a_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(b_scale_inv) & 3u)) {
    set_error("fp8_gemm_scaled: operands must be 16-byte aligned, scales 4-byte aligned");
    return FP8DP_EINVAL;
  }
  if (fa == FP8DP_E4M3 && fb == FP8DP_E4M3)
    return launch_gemm<0, 0>(a, b, M, N, K, mode, accum, a_scale_inv, b_scale_inv, y, stream);
  if (fa == FP8DP_E4M3 && fb == FP8DP_E5M2)
    return launch_gemm<0, 1>(a, b, M, N, K, mode, accum, a_scale_inv, b_scale_inv, y, stream);
  if (fa == FP8DP_E5M2 && fb == FP8DP_E4M3)
    return launch_gemm<1, 0>(a, b, M, N, K, mode, accum, a_scale_inv, b_scale_inv, y, stream);
  return launch_gemm<1, 1>(a, b, M, N, K, mode, accum, a_scale_inv, b_scale_inv, y, stream);
}
