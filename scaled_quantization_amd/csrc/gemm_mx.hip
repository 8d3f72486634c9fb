// gemm_mx.hip -- fp8_gemm_mx: the MXFP8 GEMM (E8M0 block exponents applied by
// the microscaled MFMA).  The kernel is in gemm_kernels.hpp.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace fp8dp {

template <int FA, int FB, int TN, bool EX>
static int launch_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb,
                     int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const dim3 grid((unsigned)((M / 256) * (N / (64 * TN))));
  if (K % 512 == 0 && aligned16(ea) && aligned16(eb))
    hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, false, true, false, -1, 1, 4, false, false, EX>),
                       grid, dim3(512), 0, stream, a, b, (int)M, (int)N, (int)K, nullptr, nullptr,
                       y, nullptr, 1, ea, eb);
  else
    hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, false, true, false, -1, 1, 1, false, false, EX>),
                       grid, dim3(512), 0, stream, a, b, (int)M, (int)N, (int)K, nullptr, nullptr,
                       y, nullptr, 1, ea, eb);
  return check_launch("fp8_gemm_mx");
}

template <int FA, int FB, bool EX>
static int launch_mx_tile(const uint8_t* a, const uint8_t* ea, const uint8_t* b,
                          const uint8_t* eb, int64_t M, int64_t N, int64_t K, uint16_t* y,
                          hipStream_t stream) {
  // no 256-wide tile here: with the exponent registers it would spill
  if (N % 192 == 0) return launch_mx<FA, FB, 3, EX>(a, ea, b, eb, M, N, K, y, stream);
  return launch_mx<FA, FB, 2, EX>(a, ea, b, eb, M, N, K, y, stream);
}

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int fp8_gemm_mx(const uint8_t* a, fp8dp_format fa, const uint8_t* a_scale,
                           const uint8_t* b, fp8dp_format fb, const uint8_t* b_scale, int64_t M,
                           int64_t N, int64_t K, fp8dp_accum accum, uint16_t* y,
                           hipStream_t stream) {
  if (a == nullptr || b == nullptr || y == nullptr || a_scale == nullptr || b_scale == nullptr) {
    set_error("fp8_gemm_mx: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (M < 256 || N < 128 || K < 128 || M % 256 || N % 128 || K % 128) {
    set_error("fp8_gemm_mx: M must be a positive multiple of 256, N and K of 128 (got %lld, "
              "%lld, %lld)", (long long)M, (long long)N, (long long)K);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30 ||
      (M / 256) * (N / 128) > (int64_t)0x7FFFFFFF) {
    set_error("fp8_gemm_mx: shape too large");
    return FP8DP_EINVAL;
  }
  if ((fa != FP8DP_E4M3 && fa != FP8DP_E5M2) || (fb != FP8DP_E4M3 && fb != FP8DP_E5M2) ||
      (accum != FP8DP_ACCUM_MFMA_FP8 && accum != FP8DP_ACCUM_EXACT)) {
    set_error("fp8_gemm_mx: unknown format or accumulation mode");
    return FP8DP_EINVAL;
  }
  if (!aligned16(a) || !aligned16(b) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(a_scale) & 3u) || (reinterpret_cast<uintptr_t>(b_scale) & 3u)) {
    set_error("fp8_gemm_mx: operands must be 16-byte aligned, block exponents 4-byte aligned");
    return FP8DP_EINVAL;
  }
  return dispatch_formats(fa, fb, accum, [&](auto A, auto B, auto X) {
    return launch_mx_tile<decltype(A)::value, decltype(B)::value, decltype(X)::value>(
        a, a_scale, b, b_scale, M, N, K, y, stream);
  });
}
