// gemm_kernels.hpp -- the scaled FP8 x FP8 GEMM kernels (gfx950), shared by
// the translation units that launch them (gemm.hip: forward and conditional
// GEMMs; gemm_bwd.hip: split-K and the fused squared-ReLU backward;
// gemm_mx.hip: the microscaled GEMM).
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
// (128 rows x 128 bytes each) are staged in LDS, double-buffered, with an XOR
// swizzle of the 16-byte chunks (swz() below) so the 16-byte LDS reads of 16
// consecutive rows hit distinct banks.  Global loads for the next K step are
// issued before the MFMAs of the current one.
#pragma once
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "common.hpp"
#include "gemm_core.hpp"
#include "quant_core.hpp"

#include <type_traits>

namespace fp8dp {

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

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

// The 8 codes in dwords 2Q and 2Q + 1 of an MFMA fragment as 8 FP16 values
// (byte 8Q + i -> element i; exact, as above).  An E5M2 code is the upper byte
// of the FP16 encoding of the same value (sign, 5 exponent bits with the same
// bias, 2 fraction bits; subnormals, infinities and NaN included), so it
// widens by a byte permute: each dword [b3 b2 b1 b0] gives [b1 0 b0 0] and
// [b3 0 b2 0].  E4M3 takes the hardware convert with scale 1.
template <int F, int Q>
__device__ __forceinline__ v8h_t widen8(const v8i_t& x) {
  const uint32_t d0 = (uint32_t)x[2 * Q], d1 = (uint32_t)x[2 * Q + 1];
  if constexpr (F == 1) {
    const u32x4_t r = {__builtin_amdgcn_perm(0u, d0, 0x010C000Cu),
                       __builtin_amdgcn_perm(0u, d0, 0x030C020Cu),
                       __builtin_amdgcn_perm(0u, d1, 0x010C000Cu),
                       __builtin_amdgcn_perm(0u, d1, 0x030C020Cu)};
    return __builtin_bit_cast(v8h_t, r);
  } else {
    const v2h_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    const v2h_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    const v2h_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    const v2h_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
    return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                   __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5,
                                   6, 7);
  }
}

// The same 8 codes times a power of two `scale` (2^-22 .. 2^7), widened with
// the hardware convert: exact whenever the scaled values are FP16 values,
// which the microscaled exact GEMM checks before it uses this.
template <int F, int Q>
__device__ __forceinline__ v8h_t widen8s(const v8i_t& x, float scale) {
  const uint32_t d0 = (uint32_t)x[2 * Q], d1 = (uint32_t)x[2 * Q + 1];
  v2h_t p0, p1, p2, p3;
  if constexpr (F == 1) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d0, scale, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d0, scale, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d1, scale, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d1, scale, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, scale, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, scale, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, scale, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, scale, true);
  }
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6,
                                 7);
}

// The same 8 codes times a power of two `scale`, widened to BF16 with the
// hardware convert: every code times 2^k is a BF16 value while it stays in
// BF16's normal range (measured: all 256 codes of both formats, k = -100 ..
// 100, bit for bit), which the microscaled exact GEMM ensures.
template <int F, int Q>
__device__ __forceinline__ v8bf_t widen8s_bf(const v8i_t& x, float scale) {
  const uint32_t d0 = (uint32_t)x[2 * Q], d1 = (uint32_t)x[2 * Q + 1];
  v2bf_t p0, p1, p2, p3;
  if constexpr (F == 1) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, scale, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, scale, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, scale, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, scale, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true);
  }
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6,
                                 7);
}

// Microscaled exact accumulation: each operand row's block exponents are
// folded into its BF16 widening relative to the row's largest one, value *
// 2^(e_block - e_rowmax + kMxFoldBias), and summed by the BF16 instruction
// (every code is a BF16 value; products of two have at most 8 significant
// bits, exact in FP32).  The largest block stays below 2^48 (448 * 2^39,
// 57344 * 2^32), so products stay below 2^96 and sums of up to 2^30 of them
// below 2^126; a block down to e_rowmax - kMxSpan keeps its smallest nonzero
// code at 2^-60 (E4M3: 2^(-9 + 39 - 90)) or 2^-62 (E5M2: 2^(-16 + 32 - 78)),
// so every product of two is at least 2^-122, a normal FP32 value.
template <int F> constexpr int kMxFoldBias = F == 0 ? 39 : 32;
template <int F> constexpr int kMxSpan = F == 0 ? 90 : 78;

constexpr int kBM = 128, kBN = 128;
constexpr int kGemmThreads = 256;

template <int FA, int FB, int MODE, bool EXACT>
__global__ __launch_bounds__(kGemmThreads, 2) void k_gemm(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ B, int M,
                                                          int N, int K,
                                                          const float* __restrict__ sa,
                                                          const float* __restrict__ sb,
                                                          uint16_t* __restrict__ Y,
                                                          const uint32_t* run_flag = nullptr) {
  // run_flag: the conditional GEMM's flag (a device word); zero leaves Y untouched
  if (run_flag != nullptr && *run_flag == 0u) return;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBM * kBK];
  __shared__ float lds_sa[2][kBM];

  // M may be ragged: the last row tile reads row M - 1 in place of the rows
  // past the end and does not store them
  const int tiles_n = N / kBN;
  const int ntiles = ((M + kBM - 1) / kBM) * tiles_n;
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
  auto a_row = [&](int r) { return A + (size_t)(r < M ? r : M - 1) * K + sch * 16; };
  const uint8_t* const gA0 = a_row(m0 + srow);
  const uint8_t* const gA1 = a_row(m0 + srow + 32);
  const uint8_t* const gA2 = a_row(m0 + srow + 64);
  const uint8_t* const gA3 = a_row(m0 + srow + 96);
  const uint8_t* gB = B + (size_t)(n0 + srow) * K + sch * 16;
  const size_t gstep = (size_t)32 * K;   // 256 threads / 8 chunks = 32 rows apart
  const int sa_row = (m0 + (tid & (kBM - 1))) < M ? m0 + (tid & (kBM - 1)) : M - 1;
  u32x4_t ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  float rsa = 0.0f;
#define FP8DP_GLOAD(kt)                                                                  \
  do {                                                                                   \
    const size_t k0 = (size_t)(kt) * kBK;                                                \
    ra0 = *reinterpret_cast<const u32x4_t*>(gA0 + k0);                                   \
    ra1 = *reinterpret_cast<const u32x4_t*>(gA1 + k0);                                   \
    ra2 = *reinterpret_cast<const u32x4_t*>(gA2 + k0);                                   \
    ra3 = *reinterpret_cast<const u32x4_t*>(gA3 + k0);                                   \
    rb0 = *reinterpret_cast<const u32x4_t*>(gB + k0);                                    \
    rb1 = *reinterpret_cast<const u32x4_t*>(gB + gstep + k0);                            \
    rb2 = *reinterpret_cast<const u32x4_t*>(gB + 2 * gstep + k0);                        \
    rb3 = *reinterpret_cast<const u32x4_t*>(gB + 3 * gstep + k0);                        \
    if constexpr (MODE == FP8DP_PER_GROUP128) {                                          \
      if (tid < kBM) rsa = sa[(size_t)sa_row * kgroups + (kt)];                          \
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
        if (row < M) Y[(size_t)row * N + col] = (uint16_t)bf16_rne_int(v);
      }
}

// ------------------------------------------------------------------ large tiles
// Per-tensor, MX and per-group FP8 paths for large problems.  A 512-thread workgroup (8 waves,
// two per SIMD) owns a 256 x BN tile of y (BN = 64 TN = 128, 192 or 256); wave
// w owns rows 64 (w / 2) .. +63 and columns (BN / 2)(w % 2) .. as 2 x TN tiles
// of the 32 x 32 x 64 MFMA (TN = 4 uses 252 of the 256 registers a wave may
// have at two waves per SIMD).  K advances 128 bytes per stage through a two-slot LDS
// ring.  Global memory is copied straight into LDS with
// global_load_lds_dwordx4 (no register staging): one instruction moves 64
// lanes x 16 bytes = 8 rows of 128 bytes, lane i landing at byte 16 i; lane i
// therefore fetches the global chunk of row i / 8 that swz() places at chunk
// i % 8 (the same layout as the small-tile kernel).
//
// The loop is software-pipelined by half stages, with the fragments double
// buffered: the first half of stage t reads the fragments of its second
// 64-wide k substep while the MFMAs of the first substep run; then every wave
// waits for its own copies of stage t+1, and one barrier per stage publishes
// them and shows that every wave has finished reading stage t; the second half
// refills stage t's slot with the copies of stage t+2, reads the first
// substep of stage t+1 and runs the MFMAs of stage t's second substep.  The
// copies of a stage therefore have a whole stage of MFMAs to land, and no
// LDS read waits in front of the MFMA pipe.
// The epilogue pairs adjacent output columns between neighbour lanes (one DPP
// swap) and stores BF16 pairs straight to Y.
// PG (per-128-group scales, 256 x 128 or 256 x 192 tiles): one stage is one
// 128-wide group of k, so each stage's two substeps accumulate a partial sum
// that is then promoted, acc += part * (sa[m, g] * sb[n / 128, g]) -- the
// small-tile kernel's arithmetic.  The tiles are computed transposed (B
// fragment first), which leaves one scale product per lane and fragment row
// instead of one per element: with the A rows in the registers the promotion
// cost a product per element and was slower than the small-tile kernel.
// A 192-wide tile spans two B blocks (one scale per fragment) and runs its
// stage by A fragment row rather than by substep (see the loop).
// Measured alternatives (GPT-2 shape, same tile): no half-stage pipelining
// (barrier at the stage start) about 4% slower; 64-byte stages with a 4-5
// deep ring, a 3-slot ring for A, four waves of 128 x 96, and a ping-pong of
// the two waves of each SIMD with a barrier per phase were all slower.
// SPLIT: workgroup u of (M/256)(N/BN) x splits runs split s = u' / ntiles of
// tile u' % ntiles (u' = the XCD-ordered index), over the 128-byte stages
// [s KS/splits, (s+1) KS/splits) of the KS = K/128, and writes its FP32 sums,
// unscaled, to ws[s][m][n]; k_splitk_reduce then adds the splits in order.
// MX: microscaled operands (32-value blocks along k, E8M0 block exponents
// ea [M x K/32], eb [N x K/32]).  A stage's 128 k bytes are 4 blocks, so each
// tile row needs one dword of exponents per stage: waves 0-3 copy the 256 A
// rows' dwords and waves 4-7 the B rows' into the ring slot next to the
// tiles, with the same waits and barrier.  In the 32 x 32 x 64 instruction a
// lane supplies the operand exponent of its fragment row for its 32 k bytes
// (lane / 32 selects the half), which is exactly one block: the MFMA applies
// 2^(ea - 127) 2^(eb - 127) to each block's products, and the epilogue has
// no scale to apply.
// XG = 4 (K a multiple of 512, exponent arrays 16-byte aligned): a lane's
// 4-byte exponent copy touches a row of its own, so per stage it costs as
// many cache-line requests as all the tile copies of its wave together;
// instead one 16-byte copy per row carries 4 stages' exponents, issued with
// the tiles of every fourth stage into a two-slot exponent ring (slot g % 2
// for stages 4g .. 4g+3).  Group g is issued with stage 4g, two stages before
// its first read, and its slot was last read by stage 4g - 5.
// The squared ReLU's backward applied in the epilogue (BC >= 0): the GEMM's
// output is dA, and each element leaves as the gradient code
//   code = sat_rne(bf16(two_root[c] * bf16(dA)) * scale),
//   two_root[c] = 2 sqrt(dec(c) * cache_si), c = the cached activation's code,
// i.e. exactly fp8_gemm_scaled followed by relu2_backward_quantize on its
// output, without dA's round trip through memory.
struct Relu2Bwd {
  const uint8_t* cache;     // [M x N] FP8 codes of the cached activation (format BC)
  const float* cache_si;    // the inverse scale they were cast with
  uint8_t* out;             // [M x N] gradient codes (format BF)
  const float* scale;       // the gradient state's scale
  fp8dp_acc_slot* slots;    // the gradient state's accumulators
};

// COND: the launch does nothing unless *run_flag != 0 (a device-side flag,
// e.g. the overflow mark of a scaling state), read once by every workgroup.
template <int FA, int FB, int TN, bool SPLIT, bool MX = false, bool COND = false, int BC = -1,
          int BF = 1, int XG = 1, bool PG = false, bool PER = false, bool EX = false>
__global__ __launch_bounds__(512, 1) void k_gemm_big(const uint8_t* __restrict__ A,
                                                     const uint8_t* __restrict__ B, int M, int N,
                                                     int K, const float* __restrict__ sa,
                                                     const float* __restrict__ sb,
                                                     uint16_t* __restrict__ Y,
                                                     float* __restrict__ ws, int splits,
                                                     const uint8_t* __restrict__ ea = nullptr,
                                                     const uint8_t* __restrict__ eb = nullptr,
                                                     const uint32_t* __restrict__ run_flag = nullptr,
                                                     Relu2Bwd bwd = {}) {
  static_assert(BC < 0 || !(MX || SPLIT), "the backward epilogue follows the per-tensor GEMM");
  static_assert(!(EX && MX) || TN <= 3, "exact microscaled accumulation: 256 x 128 or 256 x 192 tiles");
  if constexpr (COND) {
    if (*run_flag == 0) return;
  }
  // BC: the backward epilogue's two scalars, read before any store (read
  // later, every use after a store would wait for all stores in flight)
  float bwd_si = 0.0f, bwd_sg = 0.0f;
  if constexpr (BC >= 0) {
    bwd_si = *bwd.cache_si;
    bwd_sg = *bwd.scale;
  }
  constexpr int BM = 256, BN = 64 * TN, TM = 2;
  constexpr int ASZ = BM * kBK, TILES = (BM + BN) * kBK;   // bytes of A / of both tiles
  static_assert(XG == 1 || ((MX || PG) && XG == 4), "exponents come 1 or 4 stages per copy");
  static_assert(!(MX && SPLIT) || XG == 1, "split-K ranges need not be whole 4-stage exponent copies");
  static_assert(!PG || ((TN == 2 || TN == 3) && XG == 4 && !MX && !SPLIT && BC < 0),
                "per-group scales: 256 x 128 or 256 x 192 tiles, scales through the ring");
  static_assert(!PER || (!MX && !PG && !SPLIT && !COND && BC < 0),
                "persistent grid: the plain per-tensor path");
  constexpr bool XR = (MX || PG) && XG == 4;                // exponents / scales in their own ring
  constexpr int SLOT = TILES + (MX && !XR ? 2048 : 0);      // + 256 A and 256 B exponent dwords
  constexpr int XSZ = XR ? 8192 : 0;                        // 512 rows x 16 bytes (4 stages)
  constexpr int LA = BM / 64, LB = BN / 64;                 // tile copies per wave per stage
  constexpr int NCOPY = LA + LB + (MX && !XR ? 1 : 0);      // copies of a stage with no exponents
  constexpr int RSZ = MX && EX ? 512 : 0;                    // rows' largest block exponents
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SLOT + 2 * XSZ + RSZ];

  const int tiles_n = N / BN;
  const int ntiles = (M / BM) * tiles_n;
  // PER: a persistent grid; workgroup b runs the tiles of its passes one after
  // another through one pipeline, stage g being k-stage g % KT of the tile of
  // pass g / KT, so the next tile's first stages are copied while a tile's
  // last stage and its epilogue run
  int tile, split = 0;
  if constexpr (PER) {
    tile = tile_of_pass(blockIdx.x, 0, gridDim.x, ntiles);
  } else if constexpr (SPLIT) {
    const int u = tile_of_block(blockIdx.x, ntiles * splits);
    split = u / ntiles;
    tile = u % ntiles;
  } else {
    tile = tile_of_block(blockIdx.x, ntiles);
  }
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = (wave >> 1) * 64;
  const int wc = (wave & 1) * (BN / 2);
  // SPLIT: split s runs stages [s KS / splits, (s + 1) KS / splits) of the
  // KS = K / 128 stages (equal ranges when splits divides KS)
  const int KS = K / kBK;
  const int s0 = SPLIT ? (int)((int64_t)split * KS / splits) : 0;
  const int KT = SPLIT ? (int)((int64_t)(split + 1) * KS / splits) - s0 : KS;
  const size_t kbase = (size_t)s0 * kBK;
  const int GS = PER ? tiles_of_block(blockIdx.x, gridDim.x, ntiles) * KT : KT;   // stages to run
  if (GS == 0) return;   // (a persistent grid has no more workgroups than tiles)

  // copy instruction i of this wave covers rows 8 (wave + 8 i) .. +7; lane l
  // lands at chunk l % 8 of row l / 8 there, so it fetches the logical chunk
  // that swz() places at that position: (l % 8) ^ ((row / 2) % 8), where
  // (row / 2) % 8 = (4 wave + (l / 8) / 2) % 8 for every i
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * wave + (lrow >> 1)) & 7);
  const uint8_t* gA = A + (size_t)(m0 + wave * 8 + lrow) * K + kbase + lchunk * 16;
  const uint8_t* gB = B + (size_t)(n0 + wave * 8 + lrow) * K + kbase + lchunk * 16;
  const size_t rstep = (size_t)64 * K;
  // exponent dwords: wave w < 4 fetches A row 64 w + lane, wave w >= 4 B row
  // 64 (w - 4) + lane (clamped into the tile; the surplus dwords are unused)
  // PG: the same copies move the FP32 group scales, whose rows (K / 128
  // floats) are as long as the exponent rows: A row 64 w + lane, and for
  // waves 4-7 the tile's one row of B block scales
  const uint8_t* gE = nullptr;
  if constexpr (MX || PG) {
    const int r = (wave & 3) * 64 + lane;
    const size_t kb = (size_t)K / 32;
    if constexpr (PG) {
      // B block rows n0 / 128 and, for a 192-wide tile, n0 / 128 + 1 (lane 1 of wave 4)
      const int nbr = n0 / 128 + ((TN == 3 && r == 1) ? 1 : 0);
      gE = wave < 4 ? reinterpret_cast<const uint8_t*>(sa) + (size_t)(m0 + r) * kb
                    : reinterpret_cast<const uint8_t*>(sb) + (size_t)nbr * kb;
    }
    else
      gE = wave < 4 ? ea + (size_t)(m0 + r) * kb + kbase / 32
                    : eb + (size_t)(n0 + (r < BN ? r : BN - 1)) * kb + kbase / 32;
  }
  auto issue = [&](int kt) {
    uint8_t* base = lds + (kt & 1) * SLOT + wave * 1024;
    int64_t oa = (int64_t)kt * kBK, ob = oa;
    if constexpr (PER) {
      // the tile of stage kt, as row offsets from this workgroup's first tile
      const int t = tile_of_pass(blockIdx.x, kt / KT, gridDim.x, ntiles);
      const int64_t k0 = (int64_t)(kt % KT) * kBK;
      oa = (int64_t)((t / tiles_n) * BM - m0) * K + k0;
      ob = (int64_t)((t % tiles_n) * BN - n0) * K + k0;
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) copy16_to_lds(gA + i * rstep + oa, base + i * 8192);
#pragma unroll
    for (int i = 0; i < LB; ++i) copy16_to_lds(gB + i * rstep + ob, base + ASZ + i * 8192);
    if constexpr (XR) {
      if ((kt & 3) == 0)
        copy16_to_lds(gE + kt * 4, lds + 2 * SLOT + ((kt >> 2) & 1) * XSZ + wave * 1024);
    } else if constexpr (MX) {
      copy4_to_lds(gE + kt * 4, lds + (kt & 1) * SLOT + TILES + wave * 256);
    }
  };

  // this lane's fragment rows: A rows wr + 32 t + lane % 32, B rows wc + 32 t + lane % 32.
  // The instruction takes the 64 k of a substep as two 32-wide blocks: bytes
  // 0-15 of lane l are k 16 (l / 32) .. +15 of the first block and bytes 16-31
  // the same k of the second (measured with single-instruction probes), so
  // the lane reads 16-byte chunks h*4 + l/32 and h*4 + 2 + l/32 of substep h.
  // MX: lane l supplies the exponent of block l / 32 of its row, i.e. block
  // 2 h + l / 32 of the stage, byte 2 h + l / 32 of the row's dword; the
  // instruction reads the low byte of the scale operand.
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  auto load_frags = [&](int kt, int h, v8i_t* fa, v8i_t* fb, uint32_t* xa, uint32_t* xb) {
    const uint8_t* sA = lds + (kt & 1) * SLOT;
    const uint8_t* sB = sA + ASZ;
    const int c0 = h * 4 + fhalf;
    if constexpr (MX || PG) {
      // the row dwords of this lane's fragments (packed just before the
      // MFMAs that use them, so that no wait on these reads sits in front of
      // the MFMAs in between)
      if constexpr (XR) {
        // row r's 16 bytes at 16 r (B rows from 256 on); stage kt's dword is the (kt % 4)-th
        const uint32_t* sE =
            reinterpret_cast<const uint32_t*>(lds + 2 * SLOT + ((kt >> 2) & 1) * XSZ) + (kt & 3);
#pragma unroll
        for (int t = 0; t < TM; ++t) xa[t] = sE[4 * (wr + 32 * t + frow)];
        if constexpr (PG) {
          xb[0] = sE[4 * 256];             // the tile's B block scale (128-wide tiles)
        } else {
#pragma unroll
          for (int t = 0; t < TN; ++t) xb[t] = sE[4 * (256 + wc + 32 * t + frow)];
        }
      } else {
        const uint32_t* sE = reinterpret_cast<const uint32_t*>(sA + TILES);
#pragma unroll
        for (int t = 0; t < TM; ++t) xa[t] = sE[wr + 32 * t + frow];
#pragma unroll
        for (int t = 0; t < TN; ++t) xb[t] = sE[256 + wc + 32 * t + frow];
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int r = wr + t * 32 + frow;
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(sA + swz(r, c0));
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(sA + swz(r, c0 + 2));
      fa[t] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int r = wc + t * 32 + frow;
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(sB + swz(r, c0));
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(sB + swz(r, c0 + 2));
      fb[t] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  v16f_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // PG: the stage's partial sums (one stage = one 128-wide group), computed
  // transposed: the B fragment is the instruction's first operand, so a
  // lane holds one A row (its column lane % 32) and its 16 registers hold B
  // rows of one 128-wide B block.  The promotion then needs one product of
  // scales per lane and fragment row (sa[m] sb), not one per element.
  v16f_t part[PG && TN == 2 ? TM : 1][PG && TN == 2 ? TN : 1];
  // Without MX the scale operands are the constant 0, which the compiler
  // lowers to the unscaled instruction (checked in the generated assembly).
  auto mfmas = [&](const v8i_t* fa, const v8i_t* fb, const uint32_t* ra, const uint32_t* rb,
                   int h) {
    if constexpr (MX) {
      // the exponents of substep h packed one per byte (fragment t in byte t,
      // picked by the instruction's byte select): byte 2 h + lane / 32 of each
      // row dword
      const uint32_t bsel = 2 * h + fhalf;
      const uint32_t pair = bsel | ((bsel + 4) << 8) | 0x0C0C0000u;   // -> bytes 0, 1; 0s above
      const uint32_t xa = __builtin_amdgcn_perm(ra[1], ra[0], pair);
      const uint32_t b01 = __builtin_amdgcn_perm(rb[1], rb[0], pair);
      uint32_t xb;
      if constexpr (TN == 2) {
        xb = b01;
      } else if constexpr (TN == 3) {
        xb = __builtin_amdgcn_perm(rb[2], b01, 0x0C000100u | ((bsel + 4) << 16));
      } else {
        const uint32_t b23 = __builtin_amdgcn_perm(rb[3], rb[2], pair);
        xb = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
      }
      static_for<TM>([&](auto I) {
        static_for<TN>([&](auto J) {
          acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[I], fb[J], acc[I][J], FA, FB, decltype(I)::value, (int)xa,
              decltype(J)::value, (int)xb);
        });
      });
    } else if constexpr (PG && EX) {
      // exact: the substep as 4 FP16 instructions of 16 k each (widened codes)
      static_for<4>([&](auto Q) {
        v8h_t ha[TM], hb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) ha[i] = widen8<FA, decltype(Q)::value>(fa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) hb[j] = widen8<FB, decltype(Q)::value>(fb[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if (h == 0 && decltype(Q)::value == 0) {
              const v16f_t zero = {};
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb[j], ha[i], zero, 0, 0, 0);
            } else {
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb[j], ha[i], part[i][j], 0, 0,
                                                                  0);
            }
          }
      });
      if (h == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const float c = __uint_as_float(ra[i]) * __uint_as_float(rb[0]);
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(part[i][j][r], c, acc[i][j][r]);
        }
      }
    } else if constexpr (PG) {
      if (h == 0) {
        const v16f_t zero = {};
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], zero, FB,
                                                                        FA, 0, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], part[i][j],
                                                                        FB, FA, 0, 0, 0, 0);
        // promote with the group's scales: sa of this lane's A row, sb of the tile
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const float c = __uint_as_float(ra[i]) * __uint_as_float(rb[0]);
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(part[i][j][r], c, acc[i][j][r]);
        }
      }
    } else if constexpr (EX) {
      // exact: the substep's 64 k as 4 FP16 instructions of 16 k each, on
      // codes widened after the LDS read (the FP16 instruction multiplies
      // exactly and sums at FP32)
      static_for<4>([&](auto Q) {
        v8h_t ha[TM], hb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) ha[i] = widen8<FA, decltype(Q)::value>(fa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) hb[j] = widen8<FB, decltype(Q)::value>(fb[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[i], hb[j], acc[i][j], 0, 0, 0);
      });
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j],
                                                                     FA, FB, 0, 0, 0, 0);
    }
  };

  // MX && EX: each operand row's largest block exponent, from a scan of the
  // tile's exponent rows (thread t < 256: A row m0 + t; 256 + c: B row n0 + c)
  // into LDS; the tile folds exactly when every row's exponents span at most
  // kMxSpan binades, else it takes the unfolded fallback below.
  uint8_t* const sR = lds + 2 * SLOT + 2 * XSZ;
  int ref_a[MX && EX ? TM : 1] = {}, ref_b[MX && EX ? TN : 1] = {};
  bool mx_slow = false;
  // the 32-wide blocks this workgroup sums: all of K, or its split's range
  const int kb0 = (int)(kbase / 32), nkb = KT * (kBK / 32);
  if constexpr (MX && EX) {
    const int t = threadIdx.x, KB = K / 32;
    const uint8_t* e = t < 256 ? ea + (size_t)(m0 + t) * KB + kb0
                               : (t - 256 < BN ? eb + (size_t)(n0 + t - 256) * KB + kb0 : nullptr);
    uint32_t emax = 0, emin = 255;
    if (e != nullptr) {
      for (int k = 0; k < nkb; k += 4) {
        const uint32_t d = *reinterpret_cast<const uint32_t*>(e + k);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t v = (d >> (8 * b)) & 0xFFu;
          emax = v > emax ? v : emax;
          emin = v < emin ? v : emin;
        }
      }
      sR[t] = (uint8_t)emax;
    }
    const int span = t < 256 ? kMxSpan<FA> : kMxSpan<FB>;
    mx_slow = __syncthreads_or(e != nullptr && (int)(emax - emin) > span) != 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) ref_a[i] = sR[wr + 32 * i + frow];
#pragma unroll
    for (int j = 0; j < TN; ++j) ref_b[j] = sR[256 + wc + 32 * j + frow];
  }

  // BC >= 0: the tile's cached codes [256 x BN], row-major, copied with the
  // 16-byte global->LDS copies into the ring slot stage KT would have used
  // (free once iteration KT-2's barrier has shown every wave done with stage
  // KT-2): issued there, they have the last stage and a half to land, and the
  // last stage's wait and barrier publish them.  Copy k of wave w moves chunks
  // 64 (8 k + w) .. +63 (chunk q = row q / (BN/16), 16-byte column q % (BN/16)).
  auto issue_cache = [&](uint8_t* dst) {
    if constexpr (BC >= 0) {
      constexpr int CPR = BN / 16, NCC = BM * CPR / 512;
#pragma unroll
      for (int k = 0; k < NCC; ++k) {
        const int q = (8 * k + wave) * 64 + lane;
        copy16_to_lds(bwd.cache + (size_t)(m0 + q / CPR) * N + n0 + (q % CPR) * 16,
                      dst + (8 * k + wave) * 1024);
      }
    }
  };
  uint8_t* const cache_lds = lds + (KT & 1) * SLOT;

  // epilogue: scale, round to BF16 and store pairs of adjacent columns of the
  // tile at (tm0, tn0).  In a 32 x 32 MFMA tile the lane holds column
  // lane % 32 and register r holds row 8 (r / 4) + 4 (lane / 32) + r % 4;
  // swapping one value with the neighbour lane (DPP quad_perm 1,0,3,2) gives
  // the even lane columns (c, c+1) of row r and the odd lane the same columns
  // of row r+1.
  // MX && EX: folded sums are scaled back by 2^(rowmax_a + rowmax_b - 254 -
  // fold biases) per element (exact, ldexp); unfolded ones (the tile's exact
  // fallback) carry their block scales already
  auto epi_plain = [&](int tm0, int tn0, bool folded = true) {
    const float f = MX ? 1.0f : sa[0] * sb[0];
    const bool odd = lane & 1;
    const int colp = (lane & 31) & ~1;
    auto val = [&](int i, int j, int r) -> float {
      if constexpr (MX && EX) {
        if (!folded) return acc[i][j][r];
        const int row = wr + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        return __builtin_ldexpf(acc[i][j][r], (int)sR[row] + ref_b[j] - 254 - kMxFoldBias<FA> -
                                                  kMxFoldBias<FB>);
      } else {
        return acc[i][j][r] * f;
      }
    };
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float v0 = val(i, j, r), v1 = val(i, j, r + 1);
          const float give = odd ? v0 : v1;
          const float got = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, give), 0xB1, 0xF, 0xF,
                                                 false));
          const uint32_t packed = odd ? pack2_bf16_hw(got, v1) : pack2_bf16_hw(v0, got);
          const int row =
              tm0 + wr + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + (odd ? 1 : 0);
          const int col = tn0 + wc + j * 32 + colp;
          *reinterpret_cast<uint32_t*>(Y + (size_t)row * N + col) = packed;
        }
  };

  // SPLIT: the unscaled FP32 partial sums of this split (lanes 0-31 of a
  // store cover 32 consecutive columns); folded MX sums are scaled back first,
  // so every split's partials are in the same units
  auto split_store = [&]() {
    float* out = ws + (size_t)split * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lrow = wr + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          float v = acc[i][j][r];
          if constexpr (MX && EX) {
            if (!mx_slow)
              v = __builtin_ldexpf(v, (int)sR[lrow] + ref_b[j] - 254 - kMxFoldBias<FA> -
                                          kMxFoldBias<FB>);
          }
          out[(size_t)(m0 + lrow) * N + n0 + wc + j * 32 + (lane & 31)] = v;
        }
  };

  if constexpr (MX && EX) {
    if (mx_slow) {
      // Unfolded fallback, exact for any exponents: each wave sums every
      // 32-wide block in FP32 on its own (two FP16 instructions on the
      // widened codes, read straight from memory) and adds it to the
      // accumulator scaled by 2^(e_a + e_b - 254) -- the promotion per block
      // of the per-group path with microscaling's block size.
      const int KB = K / 32;
      for (int blk = kb0; blk < kb0 + nkb; ++blk) {
        v8h_t ha[2][TM];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const size_t k0 = (size_t)blk * 32 + 16 * sl + 8 * fhalf;
            const uint2 u = *reinterpret_cast<const uint2*>(A + (size_t)(m0 + wr + 32 * i + frow) * K + k0);
            const v8i_t x = {(int)u.x, (int)u.y, 0, 0, 0, 0, 0, 0};
            ha[sl][i] = widen8<FA, 0>(x);
          }
        // one B fragment column at a time: its TM partial sums, then their promotion
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v16f_t part[TM];
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            const size_t k0 = (size_t)blk * 32 + 16 * sl + 8 * fhalf;
            const uint2 u = *reinterpret_cast<const uint2*>(B + (size_t)(n0 + wc + 32 * j + frow) * K + k0);
            const v8i_t x = {(int)u.x, (int)u.y, 0, 0, 0, 0, 0, 0};
            const v8h_t hb = widen8<FB, 0>(x);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
              if (sl == 0) {
                const v16f_t zero = {};
                part[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[0][i], hb, zero, 0, 0, 0);
              } else {
                part[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[1][i], hb, part[i], 0, 0, 0);
              }
            }
          }
          const int e_b = eb[(size_t)(n0 + wc + 32 * j + frow) * KB + blk];
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = m0 + wr + 32 * i + (r >> 2) * 8 + fhalf * 4 + (r & 3);
              const int e_a = ea[(size_t)row * KB + blk];
              acc[i][j][r] += __builtin_ldexpf(part[i][r], e_a + e_b - 254);
            }
        }
      }
      if constexpr (SPLIT)
        split_store();
      else
        epi_plain(m0, n0, false);
      return;
    }
  }

  // prologue: stages 0 and 1 in flight, stage 0 landed and published
  issue(0);
  if (GS > 1) {
    issue(1);
    wait_vmcnt<NCOPY>();
  } else {
    wait_vmcnt<0>();
  }
  stage_barrier();
  if constexpr (PG && TN == 3) {
    // 256 x 192 tiles: the partial sums of all six fragments cannot stay live
    // across the half stage beside the accumulators, so the stage is split by
    // A fragment instead of by substep: the first half runs fragment row 0's
    // three chains (both substeps, then the promotion), the second half row
    // 1's.  Each chain is the 256 x 128 path's arithmetic -- part = B0 A0,
    // part += B1 A1, acc = fma(part, sa sb, acc) -- so the outputs are the
    // same bit for bit.  All of stage kt's B fragments and row 0's A
    // fragments are read in the previous second half, row 1's in the first
    // half, so every read of a slot is done by the barrier that frees it.
    v8i_t gb[2][TN], ga0[2], ga1[2];
    uint32_t ya0, ya1, yb[TN];
    auto read_b = [&](int kt) {
      const uint8_t* sB = lds + (kt & 1) * SLOT + ASZ;
      const uint32_t* sE =
          reinterpret_cast<const uint32_t*>(lds + 2 * SLOT + ((kt >> 2) & 1) * XSZ) + (kt & 3);
#pragma unroll
      for (int t = 0; t < TN; ++t) yb[t] = sE[4 * (256 + ((n0 + wc + 32 * t) >> 7) - (n0 >> 7))];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int r = wc + t * 32 + frow, c0 = h * 4 + fhalf;
          const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(sB + swz(r, c0));
          const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(sB + swz(r, c0 + 2));
          gb[h][t] =
              __builtin_bit_cast(v8i_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto read_a = [&](int kt, int t, v8i_t* ga, uint32_t& ya) {
      const uint8_t* sA = lds + (kt & 1) * SLOT;
      const uint32_t* sE =
          reinterpret_cast<const uint32_t*>(lds + 2 * SLOT + ((kt >> 2) & 1) * XSZ) + (kt & 3);
      const int r = wr + t * 32 + frow;
      ya = sE[4 * r];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c0 = h * 4 + fhalf;
        const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(sA + swz(r, c0));
        const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(sA + swz(r, c0 + 2));
        ga[h] = __builtin_bit_cast(v8i_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto chains = [&](const v8i_t* ga, v16f_t* p) {
      if constexpr (EX) {
        static_for<2>([&](auto H) {
          static_for<4>([&](auto Q) {
            constexpr int h = decltype(H)::value, q = decltype(Q)::value;
            const v8h_t ha = widen8<FA, q>(ga[h]);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const v8h_t hb = widen8<FB, q>(gb[h][j]);
              if constexpr (h == 0 && q == 0) {
                const v16f_t zero = {};
                p[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb, ha, zero, 0, 0, 0);
              } else {
                p[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb, ha, p[j], 0, 0, 0);
              }
            }
          });
        });
        return;
      }
      const v16f_t zero = {};
#pragma unroll
      for (int j = 0; j < TN; ++j)
        p[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[0][j], ga[0], zero, FB, FA, 0, 0,
                                                              0, 0);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        p[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[1][j], ga[1], p[j], FB, FA, 0, 0,
                                                              0, 0);
    };
    read_b(0);
    read_a(0, 0, ga0, ya0);
    for (int kt = 0; kt < GS; ++kt) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // stage kt's B and row-0 A fragments
      __builtin_amdgcn_sched_barrier(0);
      {
        v16f_t p[TN];
        chains(ga0, p);
        // row 1's reads after the instructions that read row 0's fragments
        __builtin_amdgcn_sched_barrier(0);
        read_a(kt, 1, ga1, ya1);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float c = __uint_as_float(ya0) * __uint_as_float(yb[j]);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[0][j][r] = __builtin_fmaf(p[j][r], c, acc[0][j][r]);
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[0][j]));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of stage kt are done
      wait_vmcnt<0>();                      // this wave's copies of stage kt+1 have landed
      stage_barrier();
      if (kt + 2 < GS) issue(kt + 2);
      float c1[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) c1[j] = __uint_as_float(ya1) * __uint_as_float(yb[j]);
      v16f_t p[TN];
      chains(ga1, p);
      // the next stage's reads go after the instructions that still read gb
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < GS) {
        read_b(kt + 1);
        read_a(kt + 1, 0, ga0, ya0);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[1][j][r] = __builtin_fmaf(p[j][r], c1[j], acc[1][j][r]);
    }
  } else {
    v8i_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    uint32_t xa0[TM], xb0[TN], xa1[TM], xb1[TN];   // MX: the fragments' row exponent dwords
    // EX (per tensor): the substep's 64 k run as 4 slices of 16 k on the
    // FP16 instruction.  The widened operands are double-buffered: slice
    // q + 1 (and, for the last slice, slice 0 of the substep that follows,
    // whose codes were read at the start of the half) is widened while the
    // MFMAs of slice q run, so no half starts with a run of converts in
    // front of its first MFMA, and no convert overwrites an operand an MFMA
    // in flight still reads.
    // (exact MX at 256 x 192 widens each slice just before its MFMAs: the
    // double-buffered widening's registers would spill beside the exponents)
    constexpr bool EXP = EX && !PG && !(MX && TN == 3);
    // the widened operands: FP16 (per tensor) or BF16 (microscaled: the
    // folded block exponents need its range)
    using WV = std::conditional_t<MX, v8bf_t, v8h_t>;
    auto mfma_w = [](const WV& a, const WV& b, const v16f_t& c) {
      if constexpr (MX)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
      else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    };
    WV wa[EXP ? TM : 1], wb[EXP ? TN : 1];
    // MX: slice q of substep h holds block 2 h + q / 2 of the stage (the
    // lane's bytes 0-15 are the first block's, 16-31 the second's); its codes
    // are widened times 2^(e_block - e_rowmax + kMxFoldBias), e_block from
    // the row's stage dword
    auto widen_slice = [&](const v8i_t* fa, const v8i_t* fb, const uint32_t* xa,
                           const uint32_t* xb, int h, auto Q, WV* oa, WV* ob) {
      constexpr int q = decltype(Q)::value;
      if constexpr (MX) {
        const int sh = 8 * (2 * h + q / 2);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int e = (int)((xa[i] >> sh) & 0xFFu) - ref_a[i] + kMxFoldBias<FA> + 127;
          oa[i] = widen8s_bf<FA, q>(fa[i], __uint_as_float((uint32_t)e << 23));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int e = (int)((xb[j] >> sh) & 0xFFu) - ref_b[j] + kMxFoldBias<FB> + 127;
          ob[j] = widen8s_bf<FB, q>(fb[j], __uint_as_float((uint32_t)e << 23));
        }
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) oa[i] = widen8<FA, q>(fa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) ob[j] = widen8<FB, q>(fb[j]);
      }
    };
    auto mfmas_mx_direct = [&](const v8i_t* fa, const v8i_t* fb, const uint32_t* xa,
                               const uint32_t* xb, int h) {
      static_for<4>([&](auto Q) {
        WV ha[TM], hb[TN];
        widen_slice(fa, fb, xa, xb, h, Q, ha, hb);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma_w(ha[i], hb[j], acc[i][j]);
      });
    };
    auto mfmas_ex = [&](const v8i_t* fa, const v8i_t* fb, const uint32_t* xa, const uint32_t* xb,
                        int h, const v8i_t* nfa, const v8i_t* nfb, const uint32_t* nxa,
                        const uint32_t* nxb, int nh) {
      if constexpr (EXP) {
        static_for<4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          WV na[TM], nb[TN];
          if constexpr (q < 3)
            widen_slice(fa, fb, xa, xb, h, std::integral_constant<int, q + 1>{}, na, nb);
          else
            widen_slice(nfa, nfb, nxa, nxb, nh, std::integral_constant<int, 0>{}, na, nb);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = mfma_w(wa[i], wb[j], acc[i][j]);
#pragma unroll
          for (int i = 0; i < TM; ++i) wa[i] = na[i];
#pragma unroll
          for (int j = 0; j < TN; ++j) wb[j] = nb[j];
        });
        // the half's order: its fragment reads first (their latency then
        // runs under the MFMAs), then each MFMA followed by a share of the
        // next slice's converts
        constexpr int CV = (4 * (TM + TN) + TM * TN - 1) / (TM * TN);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);
        static_for<4 * TM * TN>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, CV, 0);
        });
        // the next half's first slice stays converted in this half: without
        // a use here the compiler sinks its converts past the barrier, in
        // front of the next half's first MFMA
#pragma unroll
        for (int i = 0; i < TM; ++i) asm volatile("" : "+v"(wa[i]));
#pragma unroll
        for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(wb[j]));
      }
    };
    load_frags(0, 0, fa0, fb0, xa0, xb0);
    if constexpr (EXP) widen_slice(fa0, fb0, xa0, xb0, 0, std::integral_constant<int, 0>{}, wa, wb);
    for (int kt = 0; kt < GS; ++kt) {
      if constexpr (PG) {
        // the reads of substep 0 were issued a half stage ago: wait for them
        // here, before the reads below (else the wait covers those as well)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_sched_barrier(0);
      }
      // first half: read substep 1 of stage kt, multiply substep 0
      load_frags(kt, 1, fa1, fb1, xa1, xb1);
      if constexpr (EXP) mfmas_ex(fa0, fb0, xa0, xb0, 0, fa1, fb1, xa1, xb1, 1);
      else if constexpr (EX && MX) mfmas_mx_direct(fa0, fb0, xa0, xb0, 0);
      else mfmas(fa0, fb0, xa0, xb0, 0);
      if constexpr (MX || PG) {
        // keep these products in the first half: without a use here the
        // compiler sinks them past the barrier (they only feed later ones)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (PG && TN == 2) asm volatile("" : "+v"(part[i][j]));
            else asm volatile("" : "+v"(acc[i][j]));
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of stage kt are done
      wait_vmcnt<0>();                      // this wave's copies of stage kt+1 have landed
      stage_barrier();
      // second half: refill stage kt's slot, read substep 0 of stage kt+1, multiply substep 1
      if (kt + 2 < GS) issue(kt + 2);
      if constexpr (BC >= 0) {
        if (kt + 2 == KT) issue_cache(cache_lds);
      }
      if (kt + 1 < GS) load_frags(kt + 1, 0, fa0, fb0, xa0, xb0);
      if constexpr (EXP) mfmas_ex(fa1, fb1, xa1, xb1, 1, fa0, fb0, xa0, xb0, 0);
      else if constexpr (EX && MX) mfmas_mx_direct(fa1, fb1, xa1, xb1, 1);
      else mfmas(fa1, fb1, xa1, xb1, 1);
      if constexpr (PER) {
        if ((kt + 1) % KT == 0) {   // the last stage of a tile: its epilogue, then a fresh sum
          const int t = tile_of_pass(blockIdx.x, kt / KT, gridDim.x, ntiles);
          epi_plain((t / tiles_n) * BM, (t % tiles_n) * BN);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        }
      }
    }
  }
  if constexpr (PER) return;

  if constexpr (SPLIT) {
    split_store();
    return;
  }

  if constexpr (BC >= 0) {
    // with a single stage there was no iteration KT-2: copy now (every wave
    // has passed the stage's barrier after its last fragment reads)
    if (KT < 2) issue_cache(cache_lds);
    // 2 sqrt(dec(c) * si) for the 256 codes (threads 0-255, the per-element
    // operations of relu2_backward_quantize), in the ring slot of stage KT-1
    // (every wave passed the last stage's barrier after reading it) -- one
    // LDS array, see block_fold_in
    float* const two_root = reinterpret_cast<float*>(lds + ((KT - 1) & 1) * SLOT);
    if (threadIdx.x < 256) {
      float d;
      if constexpr (BC == 0) d = __builtin_amdgcn_cvt_pk_f32_fp8((int)threadIdx.x, false)[0];
      else d = __builtin_amdgcn_cvt_pk_f32_bf8((int)threadIdx.x, false)[0];
      two_root[threadIdx.x] = __fmul_rn(2.0f, __builtin_sqrtf(__fmul_rn(d, bwd_si)));
    }
    wait_vmcnt<0>();
    __syncthreads();
    const float f = sa[0] * sb[0];
    const float sg = bwd_sg;
    const bool odd = lane & 1;
    const int colp = (lane & 31) & ~1;
    uint32_t amax16 = 0, sat = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // per 32 x 32 tile, in three passes so that the LDS reads of its 8
        // row pairs are in flight together: (1) dA pairs and their cached
        // codes, (2) the table entries, (3) the gradient codes
        uint32_t da[8], c2[8];
        int lrow[8];
        const int lcol = wc + j * 32 + colp;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          // the pair of adjacent columns (col, col+1) of one row, as in the
          // BF16 epilogue below: dA exactly as fp8_gemm_scaled stores it
          const int r = 2 * k;
          const float v0 = acc[i][j][r] * f, v1 = acc[i][j][r + 1] * f;
          const float give = odd ? v0 : v1;
          const float got = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, give), 0xB1, 0xF, 0xF,
                                                 false));
          da[k] = odd ? pack2_bf16_hw(got, v1) : pack2_bf16_hw(v0, got);
          lrow[k] = wr + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + (odd ? 1 : 0);
          c2[k] = *reinterpret_cast<const uint16_t*>(cache_lds + lrow[k] * BN + lcol);
        }
        float t0[8], t1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          t0[k] = two_root[c2[k] & 0xFFu];
          t1[k] = two_root[c2[k] >> 8];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float g0 = __fmul_rn(t0[k], __uint_as_float(da[k] << 16));
          const float g1 = __fmul_rn(t1[k], __uint_as_float(da[k] & 0xFFFF0000u));
          const uint32_t m0g = __float_as_uint(g0) & 0x7FFFFFFFu, m1g = __float_as_uint(g1) & 0x7FFFFFFFu;
          uint32_t b, code;
          if (m0g <= kF32Inf && m1g <= kF32Inf) {
            // no NaN: the hardware conversions (the clamp saturates, the
            // convert rounds to nearest even: the integer codec's codes), and
            // the saturation count from the scaled values directly
            b = pack2_bf16_hw(g0, g1);
            const float q0 = __fmul_rn(__uint_as_float(b << 16), sg);
            const float q1 = __fmul_rn(__uint_as_float(b & 0xFFFF0000u), sg);
            code = pack2_hw<BF>(q0, q1);
            sat += saturates<BF>(q0) + saturates<BF>(q1);
          } else {
            b = pack2_bf16_int(g0, g1);
            const float q0 = __fmul_rn(__uint_as_float(b << 16), sg);
            const float q1 = __fmul_rn(__uint_as_float(b & 0xFFFF0000u), sg);
            code = enc_int<BF>(q0) | (enc_int<BF>(q1) << 8);
            sat += saturates<BF>(q0) + saturates<BF>(q1);
          }
          const uint32_t b0 = b & 0x7FFFu, b1 = (b >> 16) & 0x7FFFu;
          const uint32_t mx = b0 > b1 ? b0 : b1;
          amax16 = mx > amax16 ? mx : amax16;
          *reinterpret_cast<uint16_t*>(bwd.out + (size_t)(m0 + lrow[k]) * N + n0 + lcol) =
              (uint16_t)code;
        }
      }
    block_fold_in<512>(amax16, sat, bwd.slots,
                       reinterpret_cast<uint32_t*>(lds + ((KT - 1) & 1) * SLOT + 1024));
    return;
  }

  if constexpr (PG) {
    // transposed tiles: register r of lane l holds y[m][n] for A row
    // m = wr + 32 i + l % 32 and B row n = wc + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4,
    // so registers 4q .. 4q+3 are 4 adjacent outputs of one row: one 8-byte store
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = m0 + wr + i * 32 + (lane & 31);
          const int col = n0 + wc + j * 32 + q * 8 + (lane >> 5) * 4;
          const uint2 v = {pack2_bf16_hw(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                           pack2_bf16_hw(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
          *reinterpret_cast<uint2*>(Y + (size_t)row * N + col) = v;
        }
    return;
  }

  epi_plain(m0, n0);
}

// ------------------------------------------------------------------ host-side dispatch
// The per-tensor large-tile width for N: the widest of 192, 256, 128 that
// divides it; calls f(std::integral_constant<int, TN>).  Exact accumulation
// (EX) holds the widened operands beside the accumulators, and its 256-wide
// tile does not fit the 256 registers a wave has at two waves per SIMD
// (68-80 bytes per lane spilled), so it takes 192 or 128.
template <bool EX, typename F>
inline int with_tile_width(int64_t N, F&& f) {
  if (N % 192 == 0) return f(std::integral_constant<int, 3>{});
  if constexpr (!EX) {
    if (N % 256 == 0) return f(std::integral_constant<int, 4>{});
  }
  return f(std::integral_constant<int, 2>{});
}

// Calls f(integral_constant FA, FB, EX) for the runtime formats and accumulation mode.
template <typename F>
inline int dispatch_formats(fp8dp_format fa, fp8dp_format fb, fp8dp_accum accum, F&& f) {
  auto by_ex = [&](auto A, auto B) {
    if (accum == FP8DP_ACCUM_EXACT) return f(A, B, std::true_type{});
    return f(A, B, std::false_type{});
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (fa == FP8DP_E4M3 && fb == FP8DP_E4M3) return by_ex(I0{}, I0{});
  if (fa == FP8DP_E4M3 && fb == FP8DP_E5M2) return by_ex(I0{}, I1{});
  if (fa == FP8DP_E5M2 && fb == FP8DP_E4M3) return by_ex(I1{}, I0{});
  return by_ex(I1{}, I1{});
}

}  // namespace fp8dp
