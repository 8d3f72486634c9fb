// gemm.hip -- scaled FP8 x FP8 GEMM with FP32 accumulation and BF16 output:
// fp8_gemm_scaled (per tensor / per 128-group scales) and its conditional form
// fp8_gemm_scaled_if.  The kernels are in gemm_kernels.hpp.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace fp8dp {

template <int FA, int FB, int TN, bool EX>
static int launch_big(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                      const float* sa, const float* sb, uint16_t* y, hipStream_t stream) {
  const int64_t ntiles = (M / 256) * (N / (64 * TN));
  // more tiles than compute units and short tiles (at most 16 stages of K): a
  // persistent grid (one workgroup per CU -- the LDS ring takes more than half
  // of a CU's 160 KiB -- a multiple of 8 for the XCD order), each running its
  // tiles through one pipeline.  Measured (same outputs bit for bit): 10-14%
  // faster at K = 512-1024, 2-5% at 1536-2048, but 2-5% slower at K = 4096 and
  // beyond, where the per-tile grid's dynamic dispatch keeps the compute units
  // out of step and spreads the epilogues' store bursts
  const int64_t cus = num_cus() & ~7;
  if (cus >= 8 && ntiles > cus && K / kBK <= 16)
    hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, false, false, false, -1, 1, 1, false, true, EX>),
                       dim3((unsigned)cus), dim3(512), 0, stream, a, b, (int)M, (int)N, (int)K, sa,
                       sb, y, nullptr, 1);
  else
    hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, false, false, false, -1, 1, 1, false, false, EX>),
                       dim3((unsigned)ntiles), dim3(512), 0, stream, a, b, (int)M, (int)N, (int)K,
                       sa, sb, y, nullptr, 1);
  return check_launch("fp8_gemm_scaled");
}

template <int FA, int FB, bool EX>
static int launch_pg(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                     const float* sa, const float* sb, uint16_t* y, hipStream_t stream) {
  // 256 x 192 tiles when they take fewer rounds of the grid: one takes about
  // 1.6x as long as a 256 x 128 tile (GPT-2 shape 16384 x 768 x 3072: 256
  // tiles in one round 50.0 us against 384 in two, 62.9 us; with fewer tiles
  // than compute units the narrow tiles win, 12.8 against 17.2 us at 4096 x
  // 384 x 1024)
  // (exact accumulation: 256 x 128 only -- its 192-wide tile spills)
  const int64_t cus = num_cus();
  const int64_t t2 = (M / 256) * (N / 128), t3 = !EX && N % 192 == 0 ? (M / 256) * (N / 192) : 0;
  const int64_t r2 = (t2 + cus - 1) / cus, r3 = (t3 + cus - 1) / cus;
  if (t3 > 0 && 8 * r3 < 5 * r2)
    hipLaunchKernelGGL((k_gemm_big<FA, FB, 3, false, false, false, -1, 1, 4, true, false, false>),
                       dim3((unsigned)t3), dim3(512), 0, stream, a, b, (int)M, (int)N, (int)K, sa,
                       sb, y, nullptr, 1);
  else
    hipLaunchKernelGGL((k_gemm_big<FA, FB, 2, false, false, false, -1, 1, 4, true, false, EX>),
                       dim3((unsigned)t2), dim3(512), 0, stream, a, b, (int)M, (int)N, (int)K, sa,
                       sb, y, nullptr, 1);
  return check_launch("fp8_gemm_scaled");
}

template <int FA, int FB, int TN, bool EX>
static int launch_cond(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, uint16_t* y, const uint32_t* flag,
                       hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, false, false, true, -1, 1, 1, false, false, EX>),
                     dim3((unsigned)((M / 256) * (N / (64 * TN)))), dim3(512), 0, stream, a, b,
                     (int)M, (int)N, (int)K, sa, sb, y, nullptr, 1, nullptr, nullptr, flag);
  return check_launch("fp8_gemm_scaled_if");
}

template <int FA, int FB, int MODE, bool EXACT>
static void launch_gemm_t(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                          const float* sa, const float* sb, uint16_t* y, hipStream_t stream,
                          const uint32_t* run_flag = nullptr) {
  const unsigned blocks = (unsigned)(((M + kBM - 1) / kBM) * (N / kBN));
  hipLaunchKernelGGL((k_gemm<FA, FB, MODE, EXACT>), dim3(blocks), dim3(kGemmThreads), 0, stream,
                     a, b, (int)M, (int)N, (int)K, sa, sb, y, run_flag);
}

template <int FA, int FB, bool EX>
static int launch_gemm(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                       fp8dp_scale_mode mode, const float* sa, const float* sb, uint16_t* y,
                       hipStream_t stream) {
  // The large-tile kernels take the rows that fill whole 256-row tiles; the
  // rest (M % 256 rows, any M) go to the small-tile kernel, which masks the
  // rows past M.  Each output row comes from one kernel, so a row's value
  // does not depend on M beyond which kernel computed it.
  const int64_t Mb = M / 256 * 256;
  const bool big_t = mode == FP8DP_PER_TENSOR;
  const bool big_g = mode == FP8DP_PER_GROUP128 && K % 512 == 0 && aligned16(sa) && aligned16(sb);
  if (Mb > 0 && (big_t || big_g)) {
    int rc;
    if (big_g)
      rc = launch_pg<FA, FB, EX>(a, b, Mb, N, K, sa, sb, y, stream);
    else
      rc = with_tile_width<EX>(N, [&](auto T) {
        return launch_big<FA, FB, decltype(T)::value, EX>(a, b, Mb, N, K, sa, sb, y, stream);
      });
    if (rc != FP8DP_OK || Mb == M) return rc;
    a += Mb * K;
    y += Mb * N;
    if (big_g) sa += Mb * (K / 128);
    M -= Mb;
  }
  if (mode == FP8DP_PER_TENSOR)
    launch_gemm_t<FA, FB, FP8DP_PER_TENSOR, EX>(a, b, M, N, K, sa, sb, y, stream);
  else
    launch_gemm_t<FA, FB, FP8DP_PER_GROUP128, EX>(a, b, M, N, K, sa, sb, y, stream);
  return check_launch("fp8_gemm_scaled");
}

// fp8_gemm_scaled_if over any M: the same split of rows as launch_gemm (whole
// 256-row tiles on the large-tile kernel, the rest on the small-tile one),
// both reading the flag, so a run gives fp8_gemm_scaled's output bit for bit
template <int FA, int FB, bool EX>
static int launch_cond_rows(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, uint16_t* y, const uint32_t* flag,
                            hipStream_t stream) {
  const int64_t Mb = M / 256 * 256;
  if (Mb > 0) {
    const int rc = with_tile_width<EX>(N, [&](auto T) {
      return launch_cond<FA, FB, decltype(T)::value, EX>(a, b, Mb, N, K, sa, sb, y, flag, stream);
    });
    if (rc != FP8DP_OK || Mb == M) return rc;
  }
  launch_gemm_t<FA, FB, FP8DP_PER_TENSOR, EX>(a + Mb * K, b, M - Mb, N, K, sa, sb, y + Mb * N,
                                              stream, flag);
  return check_launch("fp8_gemm_scaled_if");
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
  if (M < 1 || N < kBN || K < kBK || N % kBN || K % kBK) {
    set_error("fp8_gemm_scaled: M must be positive, N and K positive multiples of 128 (got %lld, "
              "%lld, %lld)", (long long)M, (long long)N, (long long)K);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30 ||
      ((M + kBM - 1) / kBM) * (N / kBN) > (int64_t)0x7FFFFFFF) {
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
  return dispatch_formats(fa, fb, accum, [&](auto A, auto B, auto X) {
    return launch_gemm<decltype(A)::value, decltype(B)::value, decltype(X)::value>(
        a, b, M, N, K, mode, a_scale_inv, b_scale_inv, y, stream);
  });
}

extern "C" int fp8_gemm_scaled_if(const uint8_t* a, fp8dp_format fa, const uint8_t* b,
                                  fp8dp_format fb, int64_t M, int64_t N, int64_t K,
                                  fp8dp_accum accum, const float* a_scale_inv,
                                  const float* b_scale_inv, uint16_t* y, const uint32_t* run_flag,
                                  hipStream_t stream) {
  if (a == nullptr || b == nullptr || y == nullptr || a_scale_inv == nullptr ||
      b_scale_inv == nullptr || run_flag == nullptr) {
    set_error("fp8_gemm_scaled_if: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (M < 1 || N < 128 || K < 128 || N % 128 || K % 128) {
    set_error("fp8_gemm_scaled_if: M must be positive, N and K positive multiples of 128 (got "
              "%lld, %lld, %lld)", (long long)M, (long long)N, (long long)K);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30 ||
      ((M + 127) / 128) * (N / 128) > (int64_t)0x7FFFFFFF) {
    set_error("fp8_gemm_scaled_if: shape too large");
    return FP8DP_EINVAL;
  }
  if ((fa != FP8DP_E4M3 && fa != FP8DP_E5M2) || (fb != FP8DP_E4M3 && fb != FP8DP_E5M2) ||
      (accum != FP8DP_ACCUM_MFMA_FP8 && accum != FP8DP_ACCUM_EXACT)) {
    set_error("fp8_gemm_scaled_if: unknown format or accumulation mode");
    return FP8DP_EINVAL;
  }
  if (!aligned16(a) || !aligned16(b) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(a_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(b_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(run_flag) & 3u)) {
    set_error("fp8_gemm_scaled_if: operands must be 16-byte aligned, scales and flag 4-byte "
              "aligned");
    return FP8DP_EINVAL;
  }
  return dispatch_formats(fa, fb, accum, [&](auto A, auto B, auto X) {
    return launch_cond_rows<decltype(A)::value, decltype(B)::value, decltype(X)::value>(
        a, b, M, N, K, a_scale_inv, b_scale_inv, y, run_flag, stream);
  });
}
