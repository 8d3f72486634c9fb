// gemm_bwd.hip -- the backward GEMMs' launch forms: fp8_gemm_scaled_splitk
// (K split over workgroups, FP32 partials summed in order) and
// fp8_gemm_relu2_backward (the dgrad GEMM with the squared ReLU's backward
// and the gradient cast in its epilogue).  The kernels are in gemm_kernels.hpp.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gemm_kernels.hpp"

namespace fp8dp {

template <int BC, int BF, int TN, bool EX>
static int launch_bwd_epi(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                          const float* sa, const float* sb, uint16_t* y_unused, Relu2Bwd bwd,
                          hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_big<1, 0, TN, false, false, false, BC, BF, 1, false, false, EX>),
                     dim3((unsigned)((M / 256) * (N / (64 * TN)))), dim3(512), 0, stream, a, b,
                     (int)M, (int)N, (int)K, sa, sb, y_unused, nullptr, 1, nullptr, nullptr,
                     nullptr, bwd);
  return check_launch("fp8_gemm_relu2_backward");
}

template <int BC, int BF, bool EX>
static int launch_bwd_tile(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                           const float* sa, const float* sb, Relu2Bwd bwd, hipStream_t stream) {
  // no 256-wide tile: with the backward epilogue's registers it would spill
  if (N % 192 == 0)
    return launch_bwd_epi<BC, BF, 3, EX>(a, b, M, N, K, sa, sb, nullptr, bwd, stream);
  return launch_bwd_epi<BC, BF, 2, EX>(a, b, M, N, K, sa, sb, nullptr, bwd, stream);
}

template <int BC, int BF>
static int launch_bwd_accum(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, Relu2Bwd bwd, fp8dp_accum accum,
                            hipStream_t stream) {
  if (accum == FP8DP_ACCUM_EXACT)
    return launch_bwd_tile<BC, BF, true>(a, b, M, N, K, sa, sb, bwd, stream);
  return launch_bwd_tile<BC, BF, false>(a, b, M, N, K, sa, sb, bwd, stream);
}

// y[m, n] = bf16_rne((sum over s in order of ws[s][m][n]) * sa[0] * sb[0]), or
// without the scale product when sa is NULL (MX partials carry their block
// scales): 8 consecutive elements per thread per iteration, grid-stride.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int splits,
                                                       int64_t mn, const float* __restrict__ sa,
                                                       const float* __restrict__ sb,
                                                       uint16_t* __restrict__ y) {
  const float f = sa != nullptr ? sa[0] * sb[0] : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < mn; i += stride) {
    float v[8];
    {
      const float4 a = *reinterpret_cast<const float4*>(ws + i);
      const float4 b = *reinterpret_cast<const float4*>(ws + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    for (int s = 1; s < splits; ++s) {
      const float* p = ws + (size_t)s * mn + i;
      const float4 a = *reinterpret_cast<const float4*>(p);
      const float4 b = *reinterpret_cast<const float4*>(p + 4);
      v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
      v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
    }
    *reinterpret_cast<uint4*>(y + i) =
        make_uint4(pack2_bf16_hw(v[0] * f, v[1] * f), pack2_bf16_hw(v[2] * f, v[3] * f),
                   pack2_bf16_hw(v[4] * f, v[5] * f), pack2_bf16_hw(v[6] * f, v[7] * f));
  }
}

template <int FA, int FB, int TN, bool EX>
static int launch_split(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                        int splits, const float* sa, const float* sb, float* ws, uint16_t* y,
                        hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, true, false, false, -1, 1, 1, false, false, EX>),
                     dim3((unsigned)((M / 256) * (N / (64 * TN)) * splits)), dim3(512), 0, stream,
                     a, b, (int)M, (int)N, (int)K, sa, sb, y, ws, splits);
  if (check_launch("fp8_gemm_scaled_splitk")) return FP8DP_EHIP;
  hipLaunchKernelGGL(k_splitk_reduce, dim3(grid_for(M * N / 8, 256, 8)), dim3(256), 0, stream, ws,
                     splits, M * N, sa, sb, y);
  return check_launch("fp8_gemm_scaled_splitk");
}

template <int FA, int FB, bool EX>
static int launch_split_tile(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                             int splits, const float* sa, const float* sb, float* ws, uint16_t* y,
                             hipStream_t stream) {
  return with_tile_width<EX>(N, [&](auto T) {
    return launch_split<FA, FB, decltype(T)::value, EX>(a, b, M, N, K, splits, sa, sb, ws, y,
                                                         stream);
  });
}

template <int FA, int FB, int TN, bool EX>
static int launch_mx_split(const uint8_t* a, const uint8_t* ea, const uint8_t* b,
                           const uint8_t* eb, int64_t M, int64_t N, int64_t K, int splits,
                           float* ws, uint16_t* y, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_big<FA, FB, TN, true, true, false, -1, 1, 1, false, false, EX>),
                     dim3((unsigned)((M / 256) * (N / (64 * TN)) * splits)), dim3(512), 0, stream,
                     a, b, (int)M, (int)N, (int)K, nullptr, nullptr, y, ws, splits, ea, eb);
  if (check_launch("fp8_gemm_mx_splitk")) return FP8DP_EHIP;
  hipLaunchKernelGGL(k_splitk_reduce, dim3(grid_for(M * N / 8, 256, 8)), dim3(256), 0, stream, ws,
                     splits, M * N, nullptr, nullptr, y);
  return check_launch("fp8_gemm_mx_splitk");
}

}  // namespace fp8dp

using namespace fp8dp;

// Argument checks shared by fp8_gemm_scaled_splitk and its no-allocation form.
static int check_splitk(const char* name, const uint8_t* a, fp8dp_format fa, const uint8_t* b,
                        fp8dp_format fb, int64_t M, int64_t N, int64_t K, int32_t splits,
                        fp8dp_accum accum, const float* a_scale_inv, const float* b_scale_inv,
                        uint16_t* y) {
  if (a == nullptr || b == nullptr || y == nullptr || a_scale_inv == nullptr ||
      b_scale_inv == nullptr) {
    set_error("%s: NULL pointer argument", name);
    return FP8DP_EINVAL;
  }
  if (splits < 1 || splits > 64) {
    set_error("%s: splits must be in 1..64 (got %d)", name, (int)splits);
    return FP8DP_EINVAL;
  }
  if (M < 256 || N < 128 || K < 128 * (int64_t)splits || M % 256 || N % 128 || K % 128) {
    set_error("%s: M must be a positive multiple of 256, N and K of 128, "
              "K at least 128 * splits (got %lld, %lld, %lld, splits %d)", name, (long long)M,
              (long long)N, (long long)K, (int)splits);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30 ||
      (M / 256) * (N / 128) * splits > (int64_t)0x7FFFFFFF) {
    set_error("%s: shape too large", name);
    return FP8DP_EINVAL;
  }
  if ((fa != FP8DP_E4M3 && fa != FP8DP_E5M2) || (fb != FP8DP_E4M3 && fb != FP8DP_E5M2) ||
      (accum != FP8DP_ACCUM_MFMA_FP8 && accum != FP8DP_ACCUM_EXACT)) {
    set_error("%s: unknown format or accumulation mode", name);
    return FP8DP_EINVAL;
  }
  if (!aligned16(a) || !aligned16(b) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(a_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(b_scale_inv) & 3u)) {
    set_error("%s: operands and workspace must be 16-byte aligned, scales 4-byte aligned", name);
    return FP8DP_EINVAL;
  }
  return FP8DP_OK;
}

extern "C" int fp8_gemm_scaled_splitk(const uint8_t* a, fp8dp_format fa, const uint8_t* b,
                                      fp8dp_format fb, int64_t M, int64_t N, int64_t K,
                                      int32_t splits, fp8dp_accum accum, const float* a_scale_inv,
                                      const float* b_scale_inv, float* workspace, uint16_t* y,
                                      hipStream_t stream) {
  if (workspace == nullptr) {
    set_error("fp8_gemm_scaled_splitk: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (!aligned16(workspace)) {
    set_error("fp8_gemm_scaled_splitk: operands and workspace must be 16-byte aligned, scales "
              "4-byte aligned");
    return FP8DP_EINVAL;
  }
  const int rc = check_splitk("fp8_gemm_scaled_splitk", a, fa, b, fb, M, N, K, splits, accum,
                              a_scale_inv, b_scale_inv, y);
  if (rc != FP8DP_OK) return rc;
  return dispatch_formats(fa, fb, accum, [&](auto A, auto B, auto X) {
    return launch_split_tile<decltype(A)::value, decltype(B)::value, decltype(X)::value>(
        a, b, M, N, K, splits, a_scale_inv, b_scale_inv, workspace, y, stream);
  });
}

// ------------------------------------------------------------------ no-allocation form
// The split partials of fp8_gemm_scaled_splitk_noalloc live in this array
// (one copy per GPU, held until the process ends) instead of a caller's
// workspace.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is resolved once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
constexpr int64_t kScratchFloats = (int64_t)16 << 20;   // 64 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

static std::mutex g_scratch_mu;
static float* g_scratch_dev[64];   // per device; nullptr until resolved

// The calling thread's current device's copy of scratch (resolved on the
// first call on that device, with that device current).  The kernels run on
// the stream's device, so a stream of another device is refused: that
// device's copy of the array is at another address.
static int scratch_for_current_device(hipStream_t stream, float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    set_error("fp8_gemm_scaled_splitk_noalloc: no current HIP device (or device index >= 64)");
    return FP8DP_EHIP;
  }
  hipDevice_t sdev = -1;
  if (stream != nullptr && hipStreamGetDevice(stream, &sdev) == hipSuccess && sdev != dev) {
    set_error("fp8_gemm_scaled_splitk_noalloc: the stream belongs to device %d, the current "
              "device is %d; make the stream's device current", (int)sdev, dev);
    return FP8DP_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("fp8_gemm_scaled_splitk_noalloc: hipGetSymbolAddress failed: %s",
                hipGetErrorString(e));
      return FP8DP_EHIP;
    }
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return FP8DP_OK;
}

extern "C" int fp8_gemm_scaled_splitk_noalloc(const uint8_t* a, fp8dp_format fa,
                                              const uint8_t* b, fp8dp_format fb, int64_t M,
                                              int64_t N, int64_t K, int32_t splits,
                                              fp8dp_accum accum, const float* a_scale_inv,
                                              const float* b_scale_inv, uint16_t* y,
                                              hipStream_t stream) {
  const int rc = check_splitk("fp8_gemm_scaled_splitk_noalloc", a, fa, b, fb, M, N, K, splits,
                              accum, a_scale_inv, b_scale_inv, y);
  if (rc != FP8DP_OK) return rc;
  if ((int64_t)splits * M * N > kScratchFloats) {
    set_error("fp8_gemm_scaled_splitk_noalloc: splits * M * N = %lld floats exceeds the "
              "%lld-float (64 MiB) scratch array; use fp8_gemm_scaled_splitk with a workspace",
              (long long)splits * M * N, (long long)kScratchFloats);
    return FP8DP_EINVAL;
  }
  float* ws = nullptr;
  const int sr = scratch_for_current_device(stream, &ws);
  if (sr != FP8DP_OK) return sr;
  return dispatch_formats(fa, fb, accum, [&](auto A, auto B, auto X) {
    return launch_split_tile<decltype(A)::value, decltype(B)::value, decltype(X)::value>(
        a, b, M, N, K, splits, a_scale_inv, b_scale_inv, ws, y, stream);
  });
}

extern "C" int fp8_gemm_relu2_backward(const uint8_t* a, fp8dp_format fa, const uint8_t* b,
                                       fp8dp_format fb, int64_t M, int64_t N, int64_t K,
                                       fp8dp_accum accum, const float* a_scale_inv,
                                       const float* b_scale_inv, const uint8_t* act_cache, fp8dp_cache cache,
                                       const float* act_scale_inv, fp8dp_format fmt,
                                       fp8dp_tensor_state* st, uint8_t* dh_out,
                                       hipStream_t stream) {
  if (a == nullptr || b == nullptr || a_scale_inv == nullptr || b_scale_inv == nullptr ||
      act_cache == nullptr || act_scale_inv == nullptr || st == nullptr || dh_out == nullptr) {
    set_error("fp8_gemm_relu2_backward: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (M < 256 || N < 128 || K < 128 || M % 256 || N % 128 || K % 128) {
    set_error("fp8_gemm_relu2_backward: M must be a positive multiple of 256, N and K of 128 "
              "(got %lld, %lld, %lld)", (long long)M, (long long)N, (long long)K);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30 ||
      (M / 256) * (N / 128) > (int64_t)0x7FFFFFFF) {
    set_error("fp8_gemm_relu2_backward: shape too large");
    return FP8DP_EINVAL;
  }
  if ((fa != FP8DP_E4M3 && fa != FP8DP_E5M2) || (fb != FP8DP_E4M3 && fb != FP8DP_E5M2) ||
      (fmt != FP8DP_E4M3 && fmt != FP8DP_E5M2) ||
      (cache != FP8DP_CACHE_E4M3 && cache != FP8DP_CACHE_E5M2 && cache != FP8DP_CACHE_BF16) ||
      (accum != FP8DP_ACCUM_MFMA_FP8 && accum != FP8DP_ACCUM_EXACT)) {
    set_error("fp8_gemm_relu2_backward: unknown format, cache kind or accumulation mode");
    return FP8DP_EINVAL;
  }
  if (fa != FP8DP_E5M2 || fb != FP8DP_E4M3 || cache == FP8DP_CACHE_BF16) {
    set_error("fp8_gemm_relu2_backward: provided for E5M2 gradients x E4M3 weights with an FP8 "
              "activation cache (the FP8 recipe's dgrad)");
    return FP8DP_EUNSUPPORTED;
  }
  if (!aligned16(a) || !aligned16(b) || !aligned16(act_cache) || !aligned16(dh_out) ||
      !aligned16(st) || (reinterpret_cast<uintptr_t>(a_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(b_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(act_scale_inv) & 3u)) {
    set_error("fp8_gemm_relu2_backward: operands, cache, output and state must be 16-byte "
              "aligned, scales 4-byte aligned");
    return FP8DP_EINVAL;
  }
  const Relu2Bwd bwd{act_cache, act_scale_inv, dh_out, &st->scale, st->acc};
  const float *sa = a_scale_inv, *sb = b_scale_inv;
  if (cache == FP8DP_CACHE_E4M3)
    return fmt == FP8DP_E5M2 ? launch_bwd_accum<0, 1>(a, b, M, N, K, sa, sb, bwd, accum, stream)
                             : launch_bwd_accum<0, 0>(a, b, M, N, K, sa, sb, bwd, accum, stream);
  return fmt == FP8DP_E5M2 ? launch_bwd_accum<1, 1>(a, b, M, N, K, sa, sb, bwd, accum, stream)
                           : launch_bwd_accum<1, 0>(a, b, M, N, K, sa, sb, bwd, accum, stream);
}

extern "C" int fp8_gemm_mx_splitk(const uint8_t* a, fp8dp_format fa, const uint8_t* a_scale,
                                  const uint8_t* b, fp8dp_format fb, const uint8_t* b_scale,
                                  int64_t M, int64_t N, int64_t K, int32_t splits,
                                  fp8dp_accum accum, float* workspace, uint16_t* y,
                                  hipStream_t stream) {
  if (a_scale == nullptr || b_scale == nullptr || workspace == nullptr) {
    set_error("fp8_gemm_mx_splitk: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(a_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(b_scale) & 3u)) {
    set_error("fp8_gemm_mx_splitk: workspace must be 16-byte aligned, block exponents 4-byte "
              "aligned");
    return FP8DP_EINVAL;
  }
  // the same shape, format and alignment rules as fp8_gemm_scaled_splitk (the
  // scale arguments there are checked for NULL only: pass the exponents)
  const int rc = check_splitk("fp8_gemm_mx_splitk", a, fa, b, fb, M, N, K, splits, accum,
                              reinterpret_cast<const float*>(a_scale),
                              reinterpret_cast<const float*>(b_scale), y);
  if (rc != FP8DP_OK) return rc;
  return dispatch_formats(fa, fb, accum, [&](auto A, auto B, auto X) {
    constexpr int FA = decltype(A)::value, FB = decltype(B)::value;
    constexpr bool EX = decltype(X)::value;
    if (N % 192 == 0)
      return launch_mx_split<FA, FB, 3, EX>(a, a_scale, b, b_scale, M, N, K, splits, workspace, y,
                                            stream);
    return launch_mx_split<FA, FB, 2, EX>(a, a_scale, b, b_scale, M, N, K, splits, workspace, y,
                                          stream);
  });
}
