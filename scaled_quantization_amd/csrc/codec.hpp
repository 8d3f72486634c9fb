// codec.hpp -- device-side number-format routines for gfx950.
//
// Formats: "FP8 training: what it is and how it works", Step 1 (E4M3: 4
// exponent / 3 mantissa bits, max 448; E5M2: 5 / 2 bits, max 57344) and
// "FP8 Training & Inference", FP8 Formats.  Scale rule: the same page, Step 2
// (scale = format max / amax, applied before rounding).
//
// Two bit-exact implementations of every cast exist:
//   * integer routines (enc_*_int, bf16_rne_int) that derive each code from
//     the binary32 bit pattern -- used for slow-path elements (NaN inputs,
//     saturating vectors), ragged tails and as a selectable full codec;
//   * the gfx950 conversion instructions (v_cvt_pk_fp8_f32 /
//     v_cvt_pk_bf8_f32 / v_cvt_pk_bf16_f32) on a clamped input, 2 elements
//     per instruction.
// Both are compared against an independent CPU reference over all 2^32
// binary32 inputs by the GPU test suite.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8dp {

// Binary32 bit patterns used below.
constexpr uint32_t kF32Inf = 0x7F800000u;
constexpr uint32_t kE4M3MaxBits = 0x43E00000u;   // 448
constexpr uint32_t kE5M2MaxBits = 0x47600000u;   // 57344
constexpr uint32_t kE4M3MinNormal = 0x3C800000u; // 2^-6
constexpr uint32_t kE5M2MinNormal = 0x38800000u; // 2^-14
// A value saturates when a non-saturating round-to-nearest-even cast would
// overflow: E4M3 above 464 (the tie between 448 and the NaN step rounds to
// 448), E5M2 at or above 61440 (the tie between 57344 and 2^16 rounds to
// infinity).
constexpr uint32_t kE4M3SatAbove = 0x43E80000u;  // 464
constexpr uint32_t kE5M2SatFrom = 0x47700000u;   // 61440

template <int FMT>
struct Fmt;
template <>
struct Fmt<0> {  // E4M3
  static constexpr float maxv = 448.0f;
  static constexpr uint32_t max_code = 0x7Eu;
};
template <>
struct Fmt<1> {  // E5M2
  static constexpr float maxv = 57344.0f;
  static constexpr uint32_t max_code = 0x7Bu;
};

// ---------------------------------------------------------------- integer codec
// E4M3, saturating, round to nearest even.  Normal range: rebias the
// exponent (127 -> 7) and round the 23-bit fraction to 3 bits with the
// carry flowing into the exponent.  Below 2^-6 the spacing is 2^-9: adding
// 2^14 (whose binary32 spacing is 2^-9) rounds |v| to that grid by the FPU's
// own nearest-even rule and leaves the code in the low mantissa bits.
__device__ __forceinline__ uint32_t enc_e4m3_int(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t r = a - (120u << 23);
  const uint32_t nrm = (r + 0x7FFFFu + ((r >> 20) & 1u)) >> 20;
  const uint32_t sub = __float_as_uint(__fadd_rn(__uint_as_float(a), 16384.0f)) - 0x46800000u;
  uint32_t c = (a < kE4M3MinNormal) ? sub : nrm;
  c = (a >= kE4M3MaxBits) ? 0x7Eu : c;
  c = (a > kF32Inf) ? 0x7Fu : c;
  return c | sgn;
}

// E5M2, saturating, round to nearest even (exponent 127 -> 15, 2 fraction
// bits; below 2^-14 the spacing is 2^-16 = the binary32 spacing of 2^7).
__device__ __forceinline__ uint32_t enc_e5m2_int(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t r = a - (112u << 23);
  const uint32_t nrm = (r + 0xFFFFFu + ((r >> 21) & 1u)) >> 21;
  const uint32_t sub = __float_as_uint(__fadd_rn(__uint_as_float(a), 128.0f)) - 0x43000000u;
  uint32_t c = (a < kE5M2MinNormal) ? sub : nrm;
  c = (a >= kE5M2MaxBits) ? 0x7Bu : c;
  c = (a > kF32Inf) ? 0x7Fu : c;
  return c | sgn;
}

template <int FMT>
__device__ __forceinline__ uint32_t enc_int(float v) {
  if constexpr (FMT == 0) return enc_e4m3_int(v);
  else return enc_e5m2_int(v);
}

// BF16 round to nearest even from binary32 (returns the 16-bit pattern).
// NaN is kept (quiet bit set); overflow carries into the infinity pattern.
__device__ __forceinline__ uint32_t bf16_rne_int(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > kF32Inf) ? ((u >> 16) | 0x40u) : r;
}

template <int FMT>
__device__ __forceinline__ uint32_t saturates(float v) {
  const uint32_t a = __float_as_uint(v) & 0x7FFFFFFFu;
  if constexpr (FMT == 0) return (a > kE4M3SatAbove && a <= kF32Inf) ? 1u : 0u;
  else return (a >= kE5M2SatFrom && a <= kF32Inf) ? 1u : 0u;
}

// ---------------------------------------------------------------- hardware codec
// Four binary32 values -> four FP8 codes packed little-endian in a dword.
// The input is clamped to [-max, max] first (v_med3_f32), which is the
// saturation; the conversion instruction then rounds to nearest even.  NaN
// does not survive the clamp: callers route vectors holding NaN (and
// saturating vectors) through the integer codec instead.
template <int FMT>
__device__ __forceinline__ uint32_t pack4_hw(float v0, float v1, float v2, float v3) {
  constexpr float m = Fmt<FMT>::maxv;
  v0 = __builtin_amdgcn_fmed3f(v0, -m, m);
  v1 = __builtin_amdgcn_fmed3f(v1, -m, m);
  v2 = __builtin_amdgcn_fmed3f(v2, -m, m);
  v3 = __builtin_amdgcn_fmed3f(v3, -m, m);
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, w, true);
  }
  return (uint32_t)w;
}

// The same for two values (codes in the low 16 bits).
template <int FMT>
__device__ __forceinline__ uint32_t pack2_hw(float v0, float v1) {
  constexpr float m = Fmt<FMT>::maxv;
  v0 = __builtin_amdgcn_fmed3f(v0, -m, m);
  v1 = __builtin_amdgcn_fmed3f(v1, -m, m);
  int w;
  if constexpr (FMT == 0) w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  else w = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, 0, false);
  return (uint32_t)w & 0xFFFFu;
}

template <int FMT>
__device__ __forceinline__ uint32_t pack4_int(float v0, float v1, float v2, float v3) {
  return enc_int<FMT>(v0) | (enc_int<FMT>(v1) << 8) | (enc_int<FMT>(v2) << 16) |
         (enc_int<FMT>(v3) << 24);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two binary32 values -> packed BF16 pair (low half = lo), nearest even, using
// v_cvt_pk_bf16_f32.  Only used where the input cannot be NaN.
__device__ __forceinline__ uint32_t pack2_bf16_hw(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint32_t pack2_bf16_int(float lo, float hi) {
  return bf16_rne_int(lo) | (bf16_rne_int(hi) << 16);
}

// ---------------------------------------------------------------- decode
// FP8 code -> binary32, exact (every E4M3 / E5M2 value is a binary32 value):
// normal codes rebias the exponent (E4M3: +120, E5M2: +112) and move the
// mantissa to the top of the fraction; subnormal codes are m * 2^-9 (E4M3)
// or m * 2^-16 (E5M2); E4M3 S.1111.111 and E5M2 exponent 31 with m != 0 are
// NaN, E5M2 exponent 31 with m == 0 is infinity.
template <int FMT>
__device__ __forceinline__ float dec_int(uint32_t c) {
  const uint32_t sgn = (c & 0x80u) << 24;
  if constexpr (FMT == 0) {
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    if (e == 15u && m == 7u) return __uint_as_float(sgn | 0x7FC00000u);
    if (e == 0u) return __uint_as_float(sgn | __float_as_uint((float)m * 0x1p-9f));
    return __uint_as_float(sgn | ((e + 120u) << 23) | (m << 20));
  } else {
    const uint32_t e = (c >> 2) & 0x1Fu, m = c & 3u;
    if (e == 31u) return __uint_as_float(sgn | (m ? 0x7FC00000u : 0x7F800000u));
    if (e == 0u) return __uint_as_float(sgn | __float_as_uint((float)m * 0x1p-16f));
    return __uint_as_float(sgn | ((e + 112u) << 23) | (m << 21));
  }
}

// ---------------------------------------------------------------- scale rule
// s = max / (amax * margin) in binary32, nearest even, no contraction; falls
// back to 1 when amax * margin is not a positive finite number or the
// quotient is not finite.
__device__ __forceinline__ float scale_rule(float amax, float margin, float fmax) {
  const float d = __fmul_rn(amax, margin);
  const float s = __fdiv_rn(fmax, d);
  const bool ok = (d > 0.0f) && (__float_as_uint(d) < kF32Inf) &&
                  ((__float_as_uint(s) & 0x7FFFFFFFu) < kF32Inf);
  return ok ? s : 1.0f;
}

__device__ __forceinline__ float recip_rn(float s) { return __fdiv_rn(1.0f, s); }

// ---------------------------------------------------------------- activation
// Squared ReLU on a BF16 input held as binary32: h*h for h > 0, +0 otherwise
// (NaN and -0 included).  The product of two BF16 values is exact in binary32
// unless it overflows or falls into the binary32 subnormal range, where the
// multiply rounds to nearest even.
__device__ __forceinline__ float relu2(float x) {
  return (x > 0.0f) ? __fmul_rn(x, x) : 0.0f;
}

}  // namespace fp8dp
