// transpose.hip -- byte transpose of FP8 code matrices.
//
// The FP8 GEMM contracts along the contiguous dimension of both operands
// (y = a b^T, a [M x K], b [N x K]).  The two backward GEMMs of the FP8
// recipe ("FP8 Training & Inference", FP8 Training Recipe: E4M3 forward,
// E5M2 gradients) contract along other dimensions:
//   dX [M x K] = dY [M x N] W [N x K]      -> b = W^T    [K x N]
//   dW [N x K] = dY^T [N x M] X [M x K]    -> a = dY^T [N x M], b = X^T [K x M]
// so their operands are the cast codes transposed.  Transposing codes is
// exact (the same bytes, moved), and it keeps each tensor's scale.
//
// Kernel: a workgroup of 2 TC threads owns one 64-row x TC-byte tile (TC =
// 128 when cols allows it, else 64; no loop, the grid has a workgroup per
// tile).  Thread t loads two 16-byte row chunks (rows t / (TC/16) and 32 more,
// both loads issued first) into an LDS tile whose rows are padded to TC + 4
// bytes, an odd number of dwords.  After a barrier it takes one 8-row x
// 4-column block (rb = t % 8, cb = t / 8): eight dword reads, free of bank
// conflicts across a wave (dword (8 rb + i) (TC/4 + 1) + cb lands in bank
// 8 rb + cb + const), two 4 x 4 byte transposes of twelve byte permutes, and
// four 8-byte stores, one per destination row c0 + 4 cb + j, at source rows
// r0 + 8 rb .. +7: 8 consecutive threads write one 64-byte run.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace fp8dp {

constexpr int kTR = 64;

// bytes j of d0..d3 -> dword j (a 4 x 4 byte transpose)
__device__ __forceinline__ void t4x4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                     uint32_t* o) {
  const uint32_t a = __builtin_amdgcn_perm(d1, d0, 0x05010400u);   // d0b0 d1b0 d0b1 d1b1
  const uint32_t b = __builtin_amdgcn_perm(d1, d0, 0x07030602u);   // d0b2 d1b2 d0b3 d1b3
  const uint32_t c = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
  const uint32_t d = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
}

template <int TC>
__global__ __launch_bounds__(2 * TC) void k_transpose8(const uint8_t* __restrict__ src,
                                                       int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ dst) {
  constexpr int P = TC + 4, CPR = TC / 16, RPP = 2 * TC / CPR;   // RPP = 32 rows per pass
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTR * P];
  const int64_t tiles_c = cols / TC;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * kTR;
  const int64_t c0 = (int64_t)(blockIdx.x % tiles_c) * TC;
  const int t = threadIdx.x;
  const int rr = t / CPR, cc = t % CPR;
  uint4 v[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    v[p] = *reinterpret_cast<const uint4*>(src + (r0 + rr + RPP * p) * cols + c0 + 16 * cc);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    uint32_t* w = reinterpret_cast<uint32_t*>(tile + (rr + RPP * p) * P + 16 * cc);
    w[0] = v[p].x;
    w[1] = v[p].y;
    w[2] = v[p].z;
    w[3] = v[p].w;
  }
  __syncthreads();
  const int cb = t >> 3, rb = t & 7;
  const uint32_t* s = reinterpret_cast<const uint32_t*>(tile + (8 * rb) * P + 4 * cb);
  constexpr int PW = P / 4;
  uint32_t lo[4], hi[4];
  t4x4(s[0], s[PW], s[2 * PW], s[3 * PW], lo);
  t4x4(s[4 * PW], s[5 * PW], s[6 * PW], s[7 * PW], hi);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint2*>(dst + (c0 + 4 * cb + j) * rows + r0 + 8 * rb) =
        make_uint2(lo[j], hi[j]);
}

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int fp8_transpose(const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                             hipStream_t stream) {
  if (src == nullptr || dst == nullptr) {
    set_error("fp8_transpose: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (rows < kTR || cols < kTR || rows % kTR || cols % kTR ||
      (rows / kTR) * (cols / kTR) > (int64_t)0x7FFFFFFF) {
    set_error("fp8_transpose: rows and cols must be positive multiples of 64 (got %lld, %lld), "
              "at most 2^31 - 1 tiles of 64 x 64", (long long)rows, (long long)cols);
    return FP8DP_EINVAL;
  }
  if (!aligned16(src) || !aligned16(dst)) {
    set_error("fp8_transpose: src and dst must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  if (src == dst) {
    set_error("fp8_transpose: src and dst must not be the same buffer");
    return FP8DP_EINVAL;
  }
  if (cols % 128 == 0)
    hipLaunchKernelGGL(k_transpose8<128>, dim3((unsigned)((rows / kTR) * (cols / 128))), dim3(256),
                       0, stream, src, rows, cols, dst);
  else
    hipLaunchKernelGGL(k_transpose8<64>, dim3((unsigned)((rows / kTR) * (cols / 64))), dim3(128),
                       0, stream, src, rows, cols, dst);
  return check_launch("fp8_transpose");
}
