// quantize_t.hip -- quantize_fused (per tensor, delayed scale) that also
// writes its FP8 codes transposed, the operand layout of the weight-gradient
// GEMM.
//
// "FP8 Training & Inference", FP8 Training Recipe: the weight gradient
// dW = dY^T X is the third GEMM of a linear layer; the GEMM here contracts
// along the contiguous dimension of both operands, so it reads X's codes as
// X8^T [cols x rows] (and dY's as dY8^T).  Writing that copy from the cast's
// own registers replaces a separate transpose pass over the codes (2 bytes
// moved per code) by one more byte written per element.  The codes are the
// cast's codes: the same arithmetic as quantize_fused ("FP8 training: what it
// is and how it works", Step 2), only stored twice.
//
// Kernel (gfx950, wave64): a workgroup of 256 threads owns a 64-row x
// 128-column tile.  Thread t takes row t / 16 + 16 p (p = 0..3) and the 8
// columns 8 (t % 16) .. +7: one 16-byte load, the activation, the BF16 copy
// (16-byte store), the cast (8-byte store), exactly as quantize_fused does per
// vector, and its 8 codes into an LDS tile [64][132 bytes] (33 dwords per
// row: the transposing reads below are free of bank conflicts).  After a
// barrier each thread takes one 8-row x 4-column block, transposes it with
// twelve byte permutes, and stores 8 bytes to each of 4 rows of the
// transposed output: 8 consecutive threads cover one 64-byte run of a
// transposed row.
// Amax and saturation count fold into the state's slots once per workgroup.
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "common.hpp"
#include "quant_core.hpp"

namespace fp8dp {

constexpr int kTR = 64, kTC = 128, kTPitch = 132;

template <int FMT, int ACT, bool WBF16, bool WQ, bool HW>
__global__ __launch_bounds__(256) void k_quant_t(const uint16_t* __restrict__ h,
                                                 uint16_t* __restrict__ bout,
                                                 uint8_t* __restrict__ qout,
                                                 uint8_t* __restrict__ qt, int64_t rows,
                                                 int64_t cols, const float* __restrict__ scale_ptr,
                                                 fp8dp_acc_slot* __restrict__ slots) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTR * kTPitch];
  const float s = *scale_ptr;
  const int64_t tiles_c = cols / kTC;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * kTR;
  const int64_t c0 = (int64_t)(blockIdx.x % tiles_c) * kTC;
  const int t = threadIdx.x;
  const int rr = t >> 4, cc = t & 15;
  uint32_t amax16 = 0, sat = 0;

  uint4 x[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    x[p] = load_nt(reinterpret_cast<const uint4*>(h + (r0 + rr + 16 * p) * cols + c0 + 8 * cc));
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t off = (r0 + rr + 16 * p) * cols + c0 + 8 * cc;
    uint32_t b[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = act_pair<ACT, HW>(b[j]);
    if constexpr (WBF16) store_nt(reinterpret_cast<uint4*>(bout + off), b[0], b[1], b[2], b[3]);
    const uint32_t mx = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b);
    amax16 = mx > amax16 ? mx : amax16;
    const uint2 q = cast8<FMT, HW>(b, mx, s, sat);
    if constexpr (WQ) store_nt(reinterpret_cast<uint2*>(qout + off), q);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + (rr + 16 * p) * kTPitch + 8 * cc);
    dst[0] = q.x;
    dst[1] = q.y;
  }
  __syncthreads();

  // thread t: the 8 x 4 block of rows 8 rb .. +7 (rb = t % 8) and columns
  // 4 cb .. +3 (cb = t / 8); dword i of the block is row 8 rb + i, columns
  // 4 cb .. +3.  Two 4 x 4 byte transposes give, for column 4 cb + j, the
  // codes of the 8 rows as one 8-byte store.
  {
    const int cb = t >> 3, rb = t & 7;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + (8 * rb) * kTPitch + 4 * cb);
    constexpr int P = kTPitch / 4;
    uint32_t lo[4], hi[4];
    auto t4 = [](uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3, uint32_t* o) {
      // bytes j of d0..d3 -> dword j
      const uint32_t a = __builtin_amdgcn_perm(d1, d0, 0x05010400u);   // d0b0 d1b0 d0b1 d1b1
      const uint32_t b = __builtin_amdgcn_perm(d1, d0, 0x07030602u);   // d0b2 d1b2 d0b3 d1b3
      const uint32_t c = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
      const uint32_t d = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
      o[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
      o[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
      o[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
      o[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
    };
    t4(src[0], src[P], src[2 * P], src[3 * P], lo);
    t4(src[4 * P], src[5 * P], src[6 * P], src[7 * P], hi);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint2*>(qt + (c0 + 4 * cb + j) * rows + r0 + 8 * rb) =
          make_uint2(lo[j], hi[j]);
  }
  block_fold<256>(amax16, sat, slots);
}

template <int FMT, int ACT, bool HW>
static int launch_t(const uint16_t* h, int64_t rows, int64_t cols, uint16_t* bout, uint8_t* qout,
                    uint8_t* qt, const float* sp, fp8dp_acc_slot* slots, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows / kTR) * (cols / kTC));
#define FP8DP_LAUNCH_QT(WB, WQ)                                                                    \
  hipLaunchKernelGGL((k_quant_t<FMT, ACT, WB, WQ, HW>), dim3(grid), dim3(256), 0, stream, h, bout, \
                     qout, qt, rows, cols, sp, slots)
  if (bout && qout)
    FP8DP_LAUNCH_QT(true, true);
  else if (bout)
    FP8DP_LAUNCH_QT(true, false);
  else if (qout)
    FP8DP_LAUNCH_QT(false, true);
  else
    FP8DP_LAUNCH_QT(false, false);
#undef FP8DP_LAUNCH_QT
  return check_launch("quantize_fused_transposed");
}

template <int FMT, int ACT>
static int dispatch_t(const uint16_t* h, int64_t rows, int64_t cols, uint16_t* bout,
                      uint8_t* qout, uint8_t* qt, const float* sp, fp8dp_acc_slot* slots,
                      hipStream_t stream) {
  if (codec() == 0) return launch_t<FMT, ACT, true>(h, rows, cols, bout, qout, qt, sp, slots, stream);
  return launch_t<FMT, ACT, false>(h, rows, cols, bout, qout, qt, sp, slots, stream);
}

// ------------------------------------------------------------------ MXFP8, transposed
// quantize_mx with the blocks of 32 running down the columns, its codes and
// exponents written transposed: code^T [cols x rows], exponent^T [cols x
// rows / 32].  "FP8 training: what it is and how it works", Trade-offs and
// edge cases: one power of two per 32 adjacent values; a GEMM that contracts
// along the token dimension (the weight gradient dW = dY^T X, and the weight
// operand of dX = dY W, contracted along the output features) needs its
// blocks along that dimension.  The exponent rule and the cast are
// quantize_mx's (mx_exponent, cast8).
//
// Kernel: 256 threads own a 64-row x 128-column tile.  Thread t loads four
// 8-value row vectors (rows t / 16 + 16 p, columns 8 (t % 16) ..), applies the
// activation, stores the BF16 copy if asked, and writes the values to an LDS
// tile of 65 dwords per row.  After a barrier thread t takes the column pair
// 2 cp, 2 cp + 1 (cp = t / 4) over the 16 rows 16 rq .. (rq = t % 4): sixteen
// dword reads (dword (16 rq + i) 65 + cp lands in bank 16 rq + cp + i: free of
// conflicts across a wave, as are the row writes), byte permutes that split
// them into the two columns' 16 values, the halves' maxima swapped with the
// neighbour lane (t ^ 1 holds the other 16 rows of the block), then per
// column one exponent, 16 codes and one 16-byte store: 4 lanes write a
// 64-byte run of a transposed row.
constexpr int kMxPitchW = 65;

template <int FMT, int ACT, bool WBF16, bool HW>
__global__ __launch_bounds__(256) void k_quant_mx_t(const uint16_t* __restrict__ h,
                                                    uint16_t* __restrict__ bout,
                                                    uint8_t* __restrict__ qt,
                                                    uint8_t* __restrict__ et, int64_t rows,
                                                    int64_t cols) {
  __shared__ uint32_t tile[kTR * kMxPitchW];
  const int64_t tiles_c = cols / kTC;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * kTR;
  const int64_t c0 = (int64_t)(blockIdx.x % tiles_c) * kTC;
  const int t = threadIdx.x;
  const int rr = t >> 4, cc = t & 15;
  uint4 x[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    x[p] = load_nt(reinterpret_cast<const uint4*>(h + (r0 + rr + 16 * p) * cols + c0 + 8 * cc));
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t b[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = act_pair<ACT, HW>(b[j]);
    if constexpr (WBF16)
      store_nt(reinterpret_cast<uint4*>(bout + (r0 + rr + 16 * p) * cols + c0 + 8 * cc), b[0],
               b[1], b[2], b[3]);
    uint32_t* dst = tile + (rr + 16 * p) * kMxPitchW + 4 * cc;
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = b[j];
  }
  __syncthreads();

  const int rq = t & 3, cp = t >> 2;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = tile[(16 * rq + i) * kMxPitchW + cp];
  // column 2 cp: the low BF16 halves, rows 2 k and 2 k + 1 in dword k; column
  // 2 cp + 1: the high halves
  uint32_t col[2][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    col[0][k] = __builtin_amdgcn_perm(w[2 * k + 1], w[2 * k], 0x05040100u);
    col[1][k] = __builtin_amdgcn_perm(w[2 * k + 1], w[2 * k], 0x07060302u);
  }
  const int64_t nb = rows / 32;
  uint32_t sat = 0;   // nothing finite saturates under the block rule; unused
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t m0 = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(col[c]);
    const uint32_t m1 = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(col[c] + 4);
    uint32_t bm = m0 > m1 ? m0 : m1;
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bm, 0xB1, 0xF, 0xF, false);
    bm = o > bm ? o : bm;
    const int k = mx_exponent<FMT>(bm);
    const float mult = mx_multiplier(k);
    const uint2 q0 = cast8<FMT, HW>(col[c], m0, mult, sat);
    const uint2 q1 = cast8<FMT, HW>(col[c] + 4, m1, mult, sat);
    const int64_t dc = c0 + 2 * cp + c;
    *reinterpret_cast<uint4*>(qt + dc * rows + r0 + 16 * rq) = make_uint4(q0.x, q0.y, q1.x, q1.y);
    if ((rq & 1) == 0) et[dc * nb + r0 / 32 + rq / 2] = (uint8_t)(k + 127);
  }
}

template <int FMT, int ACT, bool HW>
static int launch_mx_t(const uint16_t* h, int64_t rows, int64_t cols, uint16_t* bout, uint8_t* qt,
                       uint8_t* et, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows / kTR) * (cols / kTC));
  if (bout)
    hipLaunchKernelGGL((k_quant_mx_t<FMT, ACT, true, HW>), dim3(grid), dim3(256), 0, stream, h,
                       bout, qt, et, rows, cols);
  else
    hipLaunchKernelGGL((k_quant_mx_t<FMT, ACT, false, HW>), dim3(grid), dim3(256), 0, stream, h,
                       bout, qt, et, rows, cols);
  return check_launch("quantize_mx_transposed");
}

template <int FMT, int ACT>
static int dispatch_mx_t(const uint16_t* h, int64_t rows, int64_t cols, uint16_t* bout,
                         uint8_t* qt, uint8_t* et, hipStream_t stream) {
  if (codec() == 0) return launch_mx_t<FMT, ACT, true>(h, rows, cols, bout, qt, et, stream);
  return launch_mx_t<FMT, ACT, false>(h, rows, cols, bout, qt, et, stream);
}

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int quantize_mx_transposed(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                                      fp8dp_format fmt, uint16_t* bf16_out, uint8_t* fp8_t_out,
                                      uint8_t* scale_t_out, hipStream_t stream) {
  if (h == nullptr || fp8_t_out == nullptr || scale_t_out == nullptr) {
    set_error("quantize_mx_transposed: h, fp8_t_out and scale_t_out must be non-NULL");
    return FP8DP_EINVAL;
  }
  if (rows < kTR || cols < kTC || rows % kTR || cols % kTC || rows > ((int64_t)1 << 31) ||
      cols > ((int64_t)1 << 31) || (rows / kTR) * (cols / kTC) > (int64_t)0x7FFFFFFF) {
    set_error("quantize_mx_transposed: rows must be a positive multiple of 64 and cols of 128 "
              "(got %lld x %lld)", (long long)rows, (long long)cols);
    return FP8DP_EINVAL;
  }
  if ((fmt != FP8DP_E4M3 && fmt != FP8DP_E5M2) ||
      (act != FP8DP_ACT_IDENTITY && act != FP8DP_ACT_RELU2)) {
    set_error("quantize_mx_transposed: unknown format %d or activation %d", (int)fmt, (int)act);
    return FP8DP_EINVAL;
  }
  if (!aligned16(h) || !aligned16(bf16_out) || !aligned16(fp8_t_out)) {
    set_error("quantize_mx_transposed: h, bf16_out and fp8_t_out must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  if (fmt == FP8DP_E4M3)
    return act == FP8DP_ACT_RELU2
               ? dispatch_mx_t<0, 1>(h, rows, cols, bf16_out, fp8_t_out, scale_t_out, stream)
               : dispatch_mx_t<0, 0>(h, rows, cols, bf16_out, fp8_t_out, scale_t_out, stream);
  return act == FP8DP_ACT_RELU2
             ? dispatch_mx_t<1, 1>(h, rows, cols, bf16_out, fp8_t_out, scale_t_out, stream)
             : dispatch_mx_t<1, 0>(h, rows, cols, bf16_out, fp8_t_out, scale_t_out, stream);
}

extern "C" int quantize_fused_transposed(const uint16_t* h, int64_t rows, int64_t cols,
                                         fp8dp_act act, fp8dp_format fmt,
                                         fp8dp_tensor_state* st, uint16_t* bf16_out,
                                         uint8_t* fp8_out, uint8_t* fp8_t_out,
                                         hipStream_t stream) {
  if (h == nullptr || st == nullptr || fp8_t_out == nullptr) {
    set_error("quantize_fused_transposed: h, st and fp8_t_out must be non-NULL");
    return FP8DP_EINVAL;
  }
  if (rows < kTR || cols < kTC || rows % kTR || cols % kTC || rows > ((int64_t)1 << 31) ||
      cols > ((int64_t)1 << 31) || (rows / kTR) * (cols / kTC) > (int64_t)0x7FFFFFFF) {
    set_error("quantize_fused_transposed: rows must be a positive multiple of 64 and cols of 128 "
              "(got %lld x %lld)", (long long)rows, (long long)cols);
    return FP8DP_EINVAL;
  }
  if ((fmt != FP8DP_E4M3 && fmt != FP8DP_E5M2) ||
      (act != FP8DP_ACT_IDENTITY && act != FP8DP_ACT_RELU2)) {
    set_error("quantize_fused_transposed: unknown format %d or activation %d", (int)fmt, (int)act);
    return FP8DP_EINVAL;
  }
  if (!aligned16(h) || !aligned16(bf16_out) || !aligned16(fp8_out) || !aligned16(fp8_t_out) ||
      !aligned16(st)) {
    set_error("quantize_fused_transposed: tensor and state pointers must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  const float* sp = &st->scale;
  fp8dp_acc_slot* slots = st->acc;
  if (fmt == FP8DP_E4M3)
    return act == FP8DP_ACT_RELU2
               ? dispatch_t<0, 1>(h, rows, cols, bf16_out, fp8_out, fp8_t_out, sp, slots, stream)
               : dispatch_t<0, 0>(h, rows, cols, bf16_out, fp8_out, fp8_t_out, sp, slots, stream);
  return act == FP8DP_ACT_RELU2
             ? dispatch_t<1, 1>(h, rows, cols, bf16_out, fp8_out, fp8_t_out, sp, slots, stream)
             : dispatch_t<1, 0>(h, rows, cols, bf16_out, fp8_out, fp8_t_out, sp, slots, stream);
}
