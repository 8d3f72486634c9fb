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
// Kernel: a 256-thread block moves 64 x 64-byte tiles: 16-byte row reads into
// LDS (rows padded to 68 bytes), then each thread gathers 16 bytes of one
// source column and writes them as 16 consecutive bytes of a destination row.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace fp8dp {

constexpr int kTile = 64, kPitch = 68;

__global__ __launch_bounds__(256) void k_transpose8(const uint8_t* __restrict__ src, int64_t rows,
                                                    int64_t cols, uint8_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kPitch];
  const int64_t tiles_c = cols / kTile;
  const int64_t ntiles = (rows / kTile) * tiles_c;
  const int lr = threadIdx.x >> 2, lq = threadIdx.x & 3;   // row / 16-byte quarter
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = (t / tiles_c) * kTile, c0 = (t % tiles_c) * kTile;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (r0 + lr) * cols + c0 + lq * 16);
    uint32_t* w = reinterpret_cast<uint32_t*>(tile + lr * kPitch + lq * 16);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
    __syncthreads();
    // destination row c0 + lr holds source column c0 + lr; this thread writes
    // its bytes for source rows r0 + 16 lq .. + 15
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t x = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x |= (uint32_t)tile[(lq * 16 + d * 4 + e) * kPitch + lr] << (8 * e);
      o[d] = x;
    }
    *reinterpret_cast<uint4*>(dst + (c0 + lr) * rows + r0 + lq * 16) =
        make_uint4(o[0], o[1], o[2], o[3]);
    __syncthreads();
  }
}

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int fp8_transpose(const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                             hipStream_t stream) {
  if (src == nullptr || dst == nullptr) {
    set_error("fp8_transpose: NULL pointer argument");
    return FP8DP_EINVAL;
  }
  if (rows < kTile || cols < kTile || rows % kTile || cols % kTile) {
    set_error("fp8_transpose: rows and cols must be positive multiples of 64 (got %lld, %lld)",
              (long long)rows, (long long)cols);
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
  const int64_t ntiles = (rows / kTile) * (cols / kTile);
  const unsigned grid = grid_for(ntiles * 256, 256, 16);
  hipLaunchKernelGGL(k_transpose8, dim3(grid), dim3(256), 0, stream, src, rows, cols, dst);
  return check_launch("fp8_transpose");
}
