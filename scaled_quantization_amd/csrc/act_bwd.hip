// act_bwd.hip -- backward of the squared ReLU from the cached activation,
// fused with the gradient's delayed-scaled FP8 cast.
//
// "FP8 training: what it is and how it works", Step 3: the activations kept
// for the backward pass may be stored in FP8 to save memory, except a few
// sensitive ones.  For A = relu(H)^2 the derivative is 2 relu(H) = 2 sqrt(A),
// so the backward needs only the cached activation -- the tensor the weight
// gradient of the down-projection reads anyway -- as its BF16 copy or as its
// FP8 codes with the inverse scale they were cast with.  Per element
// (binary32, nearest even, one operation at a time):
//   a = BF16 cache ? bf16(cache) : dec(code) * a_scale_inv
//   g = (2 sqrt(a)) * dA          (IEEE square root)
//   b = bf16_rne(g)               -> the BF16 copy of dH (optional)
//   code = sat_rne(b * s_g)       -> dH in FP8 with the gradient state's scale,
// with max |b| and the saturation count folded into that state (the same
// running accumulators as quantize_fused).
//
// Kernel: the quantizer's streaming loop -- 8 elements per lane per vector,
// two vectors in flight, non-temporal loads and stores -- reading dA (2 B per
// element) and the cache (1 or 2 B) and writing 1 (+ 2) B.
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "common.hpp"
#include "quant_core.hpp"

namespace fp8dp {

namespace {
constexpr int kThreads = 256;
// grid by read/write mix, as for the quantizer: one vector per thread with
// the BF16 dH copy (writes >= reads), 32 workgroups per CU looping without it
// (3-4 B read, 1 B written)
constexpr int kBlocksPerCU = 1 << 20;
constexpr int kBlocksPerCURead = 32;
constexpr int kCacheBf16 = FP8DP_CACHE_BF16;

typedef float v2f_t __attribute__((ext_vector_type(2)));

// The raw cache bytes of vector i (16 for BF16, 8 for FP8), loaded before
// any arithmetic so that both vectors of an iteration are in flight together.
template <int CACHE>
__device__ __forceinline__ uint4 load_cache(const void* cache, int64_t i) {
  if constexpr (CACHE == kCacheBf16) {
    return load_nt(reinterpret_cast<const uint4*>(cache) + i);
  } else {
    const uint2 c = load_nt(reinterpret_cast<const uint2*>(cache) + i);
    return make_uint4(c.x, c.y, 0u, 0u);
  }
}

// Those bytes as 8 binary32 activation values.
template <int CACHE, bool HW>
__device__ __forceinline__ void cache_values(const uint4& c, float si, float a[8]) {
  if constexpr (CACHE == kCacheBf16) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[2 * j] = __uint_as_float(w[j] << 16);
      a[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float d[4];
      if constexpr (HW) {
        v2f_t lo, hi;
        if constexpr (CACHE == 0) {
          lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[j], false);
          hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[j], true);
        } else {
          lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[j], false);
          hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[j], true);
        }
        d[0] = lo.x; d[1] = lo.y; d[2] = hi.x; d[3] = hi.y;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = dec_int<CACHE>((w[j] >> (8 * e)) & 0xFFu);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) a[4 * j + e] = __fmul_rn(d[e], si);
    }
  }
}

__device__ __forceinline__ float dgrad_elem(float a, float da) {
  const float r = __builtin_sqrtf(a);
  return __fmul_rn(__fmul_rn(2.0f, r), da);
}

template <int CACHE, int FMT, bool WBF16, bool HW, int FORM = kFormLoop>
__global__ __launch_bounds__(kThreads) void k_relu2_bwd(const uint4* __restrict__ dA,
                                                        const void* __restrict__ cache,
                                                        const float* __restrict__ a_si,
                                                        uint4* __restrict__ bout,
                                                        uint2* __restrict__ qout, int64_t n8,
                                                        int tail, const float* __restrict__ s_ptr,
                                                        fp8dp_acc_slot* __restrict__ slots) {
  const float si = CACHE == kCacheBf16 ? 1.0f : *a_si;
  const float s = *s_ptr;
  uint32_t amax16 = 0, sat = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  // An FP8 cache has 256 possible codes and one inverse scale per launch, so
  // 2 sqrt(dec(code) * si) is tabulated once per workgroup (thread t computes
  // code t with exactly the per-element operations) and each element costs
  // one LDS read and one multiply.
  __shared__ float two_root[CACHE == kCacheBf16 ? 1 : 256];
  if constexpr (CACHE != kCacheBf16) {
    static_assert(kThreads == 256, "one table entry per thread");
    float d;
    if constexpr (!HW) {
      d = dec_int<CACHE>(threadIdx.x);
    } else if constexpr (CACHE == 0) {
      d = __builtin_amdgcn_cvt_pk_f32_fp8((int)threadIdx.x, false)[0];
    } else {
      d = __builtin_amdgcn_cvt_pk_f32_bf8((int)threadIdx.x, false)[0];
    }
    two_root[threadIdx.x] = __fmul_rn(2.0f, __builtin_sqrtf(__fmul_rn(d, si)));
    __syncthreads();
  }
  auto one = [&](const uint4& d, const uint4& c, int64_t i) {
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
    float g[8];
    uint32_t gmax = 0;
    float a[8];
    if constexpr (CACHE == kCacheBf16) cache_values<CACHE, HW>(c, si, a);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (CACHE == kCacheBf16) {
        g[2 * j] = dgrad_elem(a[2 * j], __uint_as_float(dw[j] << 16));
        g[2 * j + 1] = dgrad_elem(a[2 * j + 1], __uint_as_float(dw[j] & 0xFFFF0000u));
      } else {
        const uint32_t w = j < 2 ? c.x : c.y;
        const uint32_t c0 = (w >> (16 * (j & 1))) & 0xFFu, c1 = (w >> (16 * (j & 1) + 8)) & 0xFFu;
        g[2 * j] = __fmul_rn(two_root[c0], __uint_as_float(dw[j] << 16));
        g[2 * j + 1] = __fmul_rn(two_root[c1], __uint_as_float(dw[j] & 0xFFFF0000u));
      }
      const uint32_t m0 = __float_as_uint(g[2 * j]) & 0x7FFFFFFFu;
      const uint32_t m1 = __float_as_uint(g[2 * j + 1]) & 0x7FFFFFFFu;
      gmax = m0 > gmax ? m0 : gmax;
      gmax = m1 > gmax ? m1 : gmax;
    }
    uint32_t b[4];
    // the hardware BF16 conversion is used only where no value is NaN
    if (HW && gmax <= kF32Inf) {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = pack2_bf16_hw(g[2 * j], g[2 * j + 1]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = pack2_bf16_int(g[2 * j], g[2 * j + 1]);
    }
    if constexpr (WBF16) store_nt(bout + i, b[0], b[1], b[2], b[3]);
    const uint32_t mx = vec_absmax16<true>(b);
    amax16 = mx > amax16 ? mx : amax16;
    store_nt(qout + i, cast8<FMT, HW>(b, mx, s, sat));
  };
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if constexpr (FORM == kFormOne) {
    if (i < n8) one(load_nt(dA + i), load_cache<CACHE>(cache, i), i);
  } else if constexpr (FORM == kFormPair) {
    // vectors b*2T + t and b*2T + T + t, all four loads issued first
    const int64_t i0 = (int64_t)blockIdx.x * (2 * kThreads) + threadIdx.x, i1 = i0 + kThreads;
    uint4 d0 = {}, d1 = {}, c0 = {}, c1 = {};
    if (i0 < n8) {
      d0 = load_nt(dA + i0);
      c0 = load_cache<CACHE>(cache, i0);
    }
    if (i1 < n8) {
      d1 = load_nt(dA + i1);
      c1 = load_cache<CACHE>(cache, i1);
    }
    if (i0 < n8) one(d0, c0, i0);
    if (i1 < n8) one(d1, c1, i1);
  } else {
    for (; i + stride < n8; i += 2 * stride) {
      const uint4 d0 = load_nt(dA + i), d1 = load_nt(dA + i + stride);
      const uint4 c0 = load_cache<CACHE>(cache, i), c1 = load_cache<CACHE>(cache, i + stride);
      one(d0, c0, i);
      one(d1, c1, i + stride);
    }
    if (i < n8) one(load_nt(dA + i), load_cache<CACHE>(cache, i), i);
  }
  if (tail && blockIdx.x == 0 && threadIdx.x == 0) {
    const uint16_t* dt = reinterpret_cast<const uint16_t*>(dA + n8);
    for (int t = 0; t < tail; ++t) {
      float a;
      if constexpr (CACHE == kCacheBf16) {
        a = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(cache)[n8 * 8 + t] << 16);
      } else {
        a = __fmul_rn(dec_int<CACHE>(reinterpret_cast<const uint8_t*>(cache)[n8 * 8 + t]), si);
      }
      const float gv = dgrad_elem(a, __uint_as_float((uint32_t)dt[t] << 16));
      const uint32_t bb = bf16_rne_int(gv);
      if constexpr (WBF16) reinterpret_cast<uint16_t*>(bout + n8)[t] = (uint16_t)bb;
      const uint32_t mag = bb & 0x7FFFu;
      amax16 = mag > amax16 ? mag : amax16;
      const float v = __fmul_rn(__uint_as_float(bb << 16), s);
      reinterpret_cast<uint8_t*>(qout + n8)[t] = (uint8_t)enc_int<FMT>(v);
      sat += saturates<FMT>(v);
    }
  }
  block_fold<kThreads>(amax16, sat, slots);
}

template <int CACHE, int FMT, bool WBF16>
int launch_bwd(const uint16_t* dA, const void* cache, const float* a_si, uint16_t* bout,
               uint8_t* qout, int64_t n, fp8dp_tensor_state* st, hipStream_t stream) {
  const int64_t n8 = n / 8;
  const int tail = (int)(n % 8);
  // writes at least as many bytes as it reads only with the BF16 copy and an
  // FP8 cache (3 B read, 3 B written per element)
  constexpr bool write_heavy = WBF16 && CACHE != kCacheBf16;
  const LaunchShape ls = launch_shape(n8, kThreads, write_heavy, kBlocksPerCURead);
  const unsigned grid =
      ls.form == kFormLoop || codec() != 0
          ? grid_for(n8 > 0 ? n8 : 1, kThreads, WBF16 ? kBlocksPerCU : kBlocksPerCURead)
          : ls.grid;
#define FP8DP_LAUNCH_B(F)                                                                    \
  hipLaunchKernelGGL((k_relu2_bwd<CACHE, FMT, WBF16, true, F>), dim3(grid), dim3(kThreads), 0, \
                     stream, reinterpret_cast<const uint4*>(dA), cache, a_si,                 \
                     reinterpret_cast<uint4*>(bout), reinterpret_cast<uint2*>(qout), n8, tail, \
                     &st->scale, st->acc)
  if (codec() == 0 && ls.form == kFormOne)
    FP8DP_LAUNCH_B(kFormOne);
  else if (codec() == 0 && ls.form == kFormPair)
    FP8DP_LAUNCH_B(kFormPair);
  else if (codec() == 0)
    FP8DP_LAUNCH_B(kFormLoop);
  else
    hipLaunchKernelGGL((k_relu2_bwd<CACHE, FMT, WBF16, false>), dim3(grid), dim3(kThreads), 0,
                       stream, reinterpret_cast<const uint4*>(dA), cache, a_si,
                       reinterpret_cast<uint4*>(bout), reinterpret_cast<uint2*>(qout), n8, tail,
                       &st->scale, st->acc);
#undef FP8DP_LAUNCH_B
  return check_launch("relu2_backward_quantize");
}

template <int CACHE, int FMT>
int dispatch_bwd(const uint16_t* dA, const void* cache, const float* a_si, uint16_t* bout,
                 uint8_t* qout, int64_t n, fp8dp_tensor_state* st, hipStream_t stream) {
  return bout ? launch_bwd<CACHE, FMT, true>(dA, cache, a_si, bout, qout, n, st, stream)
              : launch_bwd<CACHE, FMT, false>(dA, cache, a_si, bout, qout, n, st, stream);
}

template <int FMT>
int dispatch_cache(int cache_kind, const uint16_t* dA, const void* cache, const float* a_si,
                   uint16_t* bout, uint8_t* qout, int64_t n, fp8dp_tensor_state* st,
                   hipStream_t stream) {
  if (cache_kind == 0) return dispatch_bwd<0, FMT>(dA, cache, a_si, bout, qout, n, st, stream);
  if (cache_kind == 1) return dispatch_bwd<1, FMT>(dA, cache, a_si, bout, qout, n, st, stream);
  return dispatch_bwd<kCacheBf16, FMT>(dA, cache, a_si, bout, qout, n, st, stream);
}
}  // namespace

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int relu2_backward_quantize(const uint16_t* dA, const void* a_cache, fp8dp_cache cache,
                                       const float* a_scale_inv, int64_t rows, int64_t cols,
                                       fp8dp_format fmt, fp8dp_tensor_state* st,
                                       uint16_t* bf16_out, uint8_t* fp8_out, hipStream_t stream) {
  if (dA == nullptr || a_cache == nullptr || st == nullptr || fp8_out == nullptr || rows < 1 ||
      cols < 1) {
    set_error("relu2_backward_quantize: need non-NULL dA, a_cache, st, fp8_out and rows, "
              "cols >= 1");
    return FP8DP_EINVAL;
  }
  if (cache != FP8DP_CACHE_E4M3 && cache != FP8DP_CACHE_E5M2 && cache != FP8DP_CACHE_BF16) {
    set_error("relu2_backward_quantize: unknown cache kind %d", (int)cache);
    return FP8DP_EINVAL;
  }
  if (cache != FP8DP_CACHE_BF16 && a_scale_inv == nullptr) {
    set_error("relu2_backward_quantize: an FP8 cache needs its inverse scale");
    return FP8DP_EINVAL;
  }
  if (fmt != FP8DP_E4M3 && fmt != FP8DP_E5M2) {
    set_error("relu2_backward_quantize: unknown format %d", (int)fmt);
    return FP8DP_EINVAL;
  }
  if (!aligned16(dA) || !aligned16(a_cache) || !aligned16(bf16_out) || !aligned16(fp8_out) ||
      !aligned16(st) || (reinterpret_cast<uintptr_t>(a_scale_inv) & 3u)) {
    set_error("relu2_backward_quantize: tensors and state must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  const int64_t n = rows * cols;
  return fmt == FP8DP_E5M2
             ? dispatch_cache<1>((int)cache, dA, a_cache, a_scale_inv, bf16_out, fp8_out, n, st,
                                 stream)
             : dispatch_cache<0>((int)cache, dA, a_cache, a_scale_inv, bf16_out, fp8_out, n, st,
                                 stream);
}
