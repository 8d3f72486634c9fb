// quantize.hip -- the fused activation / BF16 copy / scaled FP8 cast / amax /
// saturation-count kernel, its per-128-group variant, the delayed-scaling
// state kernels, the weight cast, and the naive three-pass comparison kernels.
//
// Method: "Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT Records"
// (one fused kernel writes the BF16 copy, emits the FP8 copy and keeps running
// maxima without rereading the tensor; the scale is the previous step's amax
// times a safety margin), "FP8 training: what it is and how it works" (Step 2
// scale rule; Trade-offs: delayed scaling with a stored history, 1 x 128
// activation tiles and 128 x 128 weight blocks) and "FP8 Training &
// Inference" (Delayed Scaling: detect overflow).
//
// Kernel design (gfx950, wave64):
//  * one thread handles 8 BF16 values per iteration: one 16-byte load, one
//    16-byte BF16 store, one 8-byte FP8 store; grid-stride over the tensor,
//    so every byte is read once and written once;
//  * the per-vector fast path uses the hardware conversions; a vector whose
//    largest scaled magnitude could saturate (or is NaN) takes the integer
//    codec and counts saturating elements one by one -- the largest |v| of a
//    vector is fp32(max|b| * s) because rounding is monotone;
//  * per block: wave reduction with cross-lane shuffles, LDS combine, then one
//    atomic max and one atomic add into one of 64 accumulator slots of the
//    state (slot = block index mod 64, so blocks do not all hit one address).
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "common.hpp"
#include "quant_core.hpp"

namespace fp8dp {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;        // vectors of 8 per thread per loop iteration (per tensor)
// Launch form of the element-wise kernels, by their read/write mix (measured;
// launch_shape in common.hpp): kernels that write at least as many bytes as
// they read take one 8-element vector per thread with no loop (the quantizer
// with its BF16 copy, 2 B read / 3 B written: 6.4 TB/s at 0.5 and 2 GiB
// against 4.9 with 32 workgroups per CU looping); read-heavy ones take two
// vectors per thread over block-contiguous ranges with no loop.  Where the
// grid of those forms would be capped, the grid-stride loop runs over
// kBlocksPerCU / kBlocksPerCURead workgroups per CU (the best of a sweep of
// 8-96 for the loop with reads > writes).
constexpr int kBlocksPerCU = 1 << 20;  // writes >= reads: no cap below one vector per thread
constexpr int kBlocksPerCURead = 32;   // reads > writes


// ------------------------------------------------------------------ per tensor
// h/bout/qout are viewed as vectors of 8 elements (n8 of them); the last
// `tail` elements (n % 8) are handled by thread 0 of block 0 with the scalar
// routine.  scale_ptr: the multiplier (read once); slots: accumulators or
// nullptr.  FORM: kFormOne / kFormPair (the grid covers every vector, one or
// two per thread, loaded first thing, no loop) or kFormLoop (grid-stride).
// UPD: the launch also closes the step (block_fold_update): slots are st->acc.
template <int FMT, int ACT, bool WBF16, bool AMAX, bool CAST, bool HW, int FORM = kFormLoop,
          bool UPD = false>
__global__ __launch_bounds__(kThreads) void k_quant_tensor(
    const uint4* __restrict__ h, uint4* __restrict__ bout, uint2* __restrict__ qout, int64_t n8,
    int tail, const float* __restrict__ scale_ptr, fp8dp_acc_slot* __restrict__ slots,
    fp8dp_tensor_state* st = nullptr) {
  const float s = CAST ? *scale_ptr : 1.0f;
  uint32_t amax16 = 0, sat = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto one = [&](const uint4& x, int64_t i) {
    uint32_t b[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = act_pair<ACT, HW>(b[j]);
    if constexpr (WBF16) store_nt(bout + i, b[0], b[1], b[2], b[3]);
    const uint32_t mx = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b);
    if constexpr (AMAX) amax16 = mx > amax16 ? mx : amax16;
    if constexpr (CAST) store_nt(qout + i, cast8<FMT, HW>(b, mx, s, sat));
  };
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if constexpr (FORM == kFormOne) {
    if (i < n8) one(load_nt(h + i), i);
  } else if constexpr (FORM == kFormPair) {
    const int64_t i0 = (int64_t)blockIdx.x * (2 * kThreads) + threadIdx.x, i1 = i0 + kThreads;
    uint4 x0 = {}, x1 = {};
    if (i0 < n8) x0 = load_nt(h + i0);
    if (i1 < n8) x1 = load_nt(h + i1);
    if (i0 < n8) one(x0, i0);
    if (i1 < n8) one(x1, i1);
  } else {
    // kUnroll grid-strided vectors per iteration, all loads issued first: more
    // bytes in flight per thread to cover HBM latency
    for (; i + (kUnroll - 1) * stride < n8; i += kUnroll * stride) {
      uint4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = load_nt(h + i + u * stride);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) one(x[u], i + u * stride);
    }
    for (; i < n8; i += stride) one(load_nt(h + i), i);
  }
  if (tail && blockIdx.x == 0 && threadIdx.x == 0) {
    const uint16_t* ht = reinterpret_cast<const uint16_t*>(h + n8);
    for (int t = 0; t < tail; ++t) {
      uint16_t bb;
      uint8_t q;
      uint32_t a16 = 0;
      quant_one<FMT, ACT>(ht[t], s, bb, q, a16, sat);
      if constexpr (WBF16) reinterpret_cast<uint16_t*>(bout + n8)[t] = bb;
      if constexpr (CAST) reinterpret_cast<uint8_t*>(qout + n8)[t] = q;
      if constexpr (AMAX) amax16 = a16 > amax16 ? a16 : amax16;
    }
  }
  if constexpr (UPD) {
    __shared__ uint32_t sm[2 * (kThreads / 64)];
    block_fold_update<kThreads>(amax16, sat, st, sm);
  } else if (slots != nullptr && (AMAX || CAST)) {
    block_fold<kThreads>(AMAX ? amax16 : 0u, CAST ? sat : 0u, slots);
  }
}

// ------------------------------------------------------------------ per group
// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15): quad swaps, then
// the half-row and row mirrors.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  uint32_t o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
  v = o > v ? o : v;
  return v;
}

// Each group of 128 elements is 16 vectors, handled by the 16 lanes of one
// DPP row (the grid stride is a multiple of 16 and n8 % 16 == 0, so a row is
// active or inactive as a whole).  Current scaling: s_g = max / amax_g.
template <int FMT, int ACT, bool WBF16, bool WFP8, bool ACC, bool HW, int FORM = kFormLoop>
__global__ __launch_bounds__(kThreads) void k_quant_group(
    const uint4* __restrict__ h, uint4* __restrict__ bout, uint2* __restrict__ qout,
    float* __restrict__ gsi, int64_t n8, fp8dp_acc_slot* __restrict__ slots) {
  uint32_t amax16 = 0, sat = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto one = [&](const uint4& x, int64_t i) {
    uint32_t b[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = act_pair<ACT, HW>(b[j]);
    if constexpr (WBF16) store_nt(bout + i, b[0], b[1], b[2], b[3]);
    const uint32_t mx = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b);
    const uint32_t gmax = row16_max(mx);
    amax16 = gmax > amax16 ? gmax : amax16;
    if constexpr (WFP8) {
      const float sg = scale_rule(__uint_as_float(gmax << 16), 1.0f, Fmt<FMT>::maxv);
      if ((threadIdx.x & 15) == 0) gsi[i >> 4] = recip_rn(sg);
      store_nt(qout + i, cast8<FMT, HW>(b, mx, sg, sat));
    }
  };
  // the loop takes two grid-strided vectors per iteration (the stride is a
  // multiple of 16, so each DPP row still holds one whole group); the pair
  // form's two ranges start at multiples of 16 vectors likewise
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if constexpr (FORM == kFormPair) {
    const int64_t i0 = (int64_t)blockIdx.x * (2 * kThreads) + threadIdx.x, i1 = i0 + kThreads;
    uint4 x0 = {}, x1 = {};
    if (i0 < n8) x0 = load_nt(h + i0);
    if (i1 < n8) x1 = load_nt(h + i1);
    if (i0 < n8) one(x0, i0);
    if (i1 < n8) one(x1, i1);
  } else {
    if constexpr (FORM == kFormLoop) {
      for (; i + stride < n8; i += 2 * stride) {
        const uint4 x0 = load_nt(h + i), x1 = load_nt(h + i + stride);
        one(x0, i);
        one(x1, i + stride);
      }
    }
    if (i < n8) one(load_nt(h + i), i);
  }
  if constexpr (ACC) block_fold<kThreads>(amax16, sat, slots);
}

// ------------------------------------------------------------------ recompute on overflow
// "FP8 Training & Inference", Delayed Scaling: when the delayed scale was too
// large the step is detected and recomputed with a corrected scale.  Launched
// after amax_history_update: if that update flagged the step (overflow != 0)
// every element is cast again with the state's new scale (which includes the
// step's own amax); otherwise every block returns at once.  The BF16 copy
// does not depend on the scale and is not rewritten; nothing is folded into
// the accumulators (the step's amax is already in the history).
template <int FMT, int ACT, bool HW>
__global__ __launch_bounds__(kThreads) void k_quant_recast(const uint4* __restrict__ h,
                                                           uint2* __restrict__ qout, int64_t n8,
                                                           int tail,
                                                           const fp8dp_tensor_state* __restrict__ st) {
  if (st->overflow == 0) return;
  const float s = st->scale;
  uint32_t sat = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    const uint4 x = load_nt(h + i);
    uint32_t b[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = act_pair<ACT, HW>(b[j]);
    store_nt(qout + i, cast8<FMT, HW>(b, vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b), s, sat));
  }
  if (tail && blockIdx.x == 0 && threadIdx.x == 0) {
    const uint16_t* ht = reinterpret_cast<const uint16_t*>(h + n8);
    for (int t = 0; t < tail; ++t) {
      uint16_t bb;
      uint8_t q;
      uint32_t a16 = 0;
      quant_one<FMT, ACT>(ht[t], s, bb, q, a16, sat);
      reinterpret_cast<uint8_t*>(qout + n8)[t] = q;
    }
  }
}

// ------------------------------------------------------------------ MXFP8
// The block exponent rule (mx_exponent, mx_multiplier) is in quant_core.hpp.

// Each block of 32 is 4 vectors of 8, held by the 4 lanes of a DPP quad (the
// grid stride is a multiple of 4 and n8 % 4 == 0, so a quad is active or
// inactive as a whole); two quad swaps give every lane the block maximum, and
// the quad's first lane writes the exponent byte.
template <int FMT, int ACT, bool WBF16, bool HW, int FORM = kFormLoop>
__global__ __launch_bounds__(kThreads) void k_quant_mx(const uint4* __restrict__ h,
                                                       uint4* __restrict__ bout,
                                                       uint2* __restrict__ qout,
                                                       uint8_t* __restrict__ e8, int64_t n8) {
  uint32_t sat = 0;   // nothing finite saturates under this rule; the count is unused
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto one = [&](const uint4& x, int64_t i) {
    uint32_t b[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = act_pair<ACT, HW>(b[j]);
    if constexpr (WBF16) store_nt(bout + i, b[0], b[1], b[2], b[3]);
    const uint32_t mx = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b);
    uint32_t bm = mx;
    uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bm, 0xB1, 0xF, 0xF, false);
    bm = o > bm ? o : bm;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bm, 0x4E, 0xF, 0xF, false);
    bm = o > bm ? o : bm;
    const int k = mx_exponent<FMT>(bm);
    if ((threadIdx.x & 3) == 0) e8[i >> 2] = (uint8_t)(k + 127);
    store_nt(qout + i, cast8<FMT, HW>(b, mx, mx_multiplier(k), sat));
  };
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // one or two vectors per thread without a loop (n8 % 4 == 0 and ranges that
  // start at multiples of 4 vectors keep quads whole)
  if constexpr (FORM == kFormOne) {
    if (i < n8) one(load_nt(h + i), i);
    return;
  } else if constexpr (FORM == kFormPair) {
    const int64_t i0 = (int64_t)blockIdx.x * (2 * kThreads) + threadIdx.x, i1 = i0 + kThreads;
    uint4 x0 = {}, x1 = {};
    if (i0 < n8) x0 = load_nt(h + i0);
    if (i1 < n8) x1 = load_nt(h + i1);
    if (i0 < n8) one(x0, i0);
    if (i1 < n8) one(x1, i1);
    return;
  }
  for (; i + (kUnroll - 1) * stride < n8; i += kUnroll * stride) {
    uint4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = load_nt(h + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) one(x[u], i + u * stride);
  }
  for (; i < n8; i += stride) one(load_nt(h + i), i);
}

// ------------------------------------------------------------------ state
__global__ void k_state_init(fp8dp_tensor_state* st, int fmt, int hist_len, float margin,
                             float initial_amax) {
  const int l = threadIdx.x;  // 64 threads
  st->acc[l].amax = 0;
  st->acc[l].ticket = 0;
  st->acc[l].sat = 0;
  if (l < FP8DP_MAX_HIST) st->history[l] = (l < hist_len) ? initial_amax : 0.0f;
  if (l == 0) {
    const float hm = __uint_as_float(__float_as_uint(initial_amax) & 0x7FFFFFFFu);
    const float s = scale_rule(hm, margin, fmt == 0 ? 448.0f : 57344.0f);
    st->scale = s;
    st->scale_inv = recip_rn(s);
    st->scale_inv_used = st->scale_inv;
    st->overflow = 0;
    st->sat_last = 0;
    st->amax_last = 0.0f;
    st->margin = margin;
    st->hist_len = hist_len;
    st->hist_pos = 0;
    st->steps = 0;
    st->fmt = fmt;
    st->ticket = 0;
  }
}

// One wave closes the step (state_update_wave, quant_core.hpp).
__global__ void k_history_update(fp8dp_tensor_state* st) { state_update_wave(st); }

// ------------------------------------------------------------------ weights
__global__ void k_w_zero(float* scale_out) { scale_out[1] = 0.0f; }

__global__ __launch_bounds__(kThreads) void k_w_amax(const uint4* __restrict__ w, int64_t n8,
                                                     int tail, uint32_t* __restrict__ amax_bits) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    const uint4 x = w[i];
    const uint32_t b[4] = {x.x, x.y, x.z, x.w};
    const uint32_t mx = vec_absmax16<true>(b);
    m = mx > m ? mx : m;
  }
  if (tail && blockIdx.x == 0 && threadIdx.x == 0) {
    const uint16_t* t = reinterpret_cast<const uint16_t*>(w + n8);
    for (int k = 0; k < tail; ++k) {
      const uint32_t mag = t[k] & 0x7FFFu;
      m = mag > m ? mag : m;
    }
  }
  __shared__ uint32_t s_max[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) m = s_max[i] > m ? s_max[i] : m;
    m = s_max[0] > m ? s_max[0] : m;
    if (m) atomicMax(amax_bits, m << 16);
  }
}

template <int FMT>
__global__ void k_w_final(float* scale_out) {
  const float amax = scale_out[1];
  const float s = scale_rule(amax, 1.0f, Fmt<FMT>::maxv);
  scale_out[0] = recip_rn(s);
  scale_out[1] = s;
}

// One 128 x 128 block per workgroup: thread t holds row t/2, columns
// 64*(t%2) .. +64 (8 vectors) in registers, so the block is read once.
template <int FMT, bool HW>
__global__ __launch_bounds__(kThreads) void k_w_block(const uint16_t* __restrict__ w, int64_t K,
                                                      uint8_t* __restrict__ w8,
                                                      float* __restrict__ scale_out) {
  const int64_t kb = K / 128;
  const int64_t bi = blockIdx.x / kb, bj = blockIdx.x % kb;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t off = (bi * 128 + r) * K + bj * 128 + half * 64;
  const uint4* src = reinterpret_cast<const uint4*>(w + off);
  uint32_t b[8][4];
  uint32_t mx[8];
  uint32_t m = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint4 x = src[v];
    b[v][0] = x.x; b[v][1] = x.y; b[v][2] = x.z; b[v][3] = x.w;
    mx[v] = vec_absmax16<true>(b[v]);
    m = mx[v] > m ? mx[v] : m;
  }
  __shared__ uint32_t s_max[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t t = __shfl_xor(m, o);
    m = t > m ? t : m;
  }
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) m = s_max[i] > m ? s_max[i] : m;
  const float s = scale_rule(__uint_as_float(m << 16), 1.0f, Fmt<FMT>::maxv);
  if (threadIdx.x == 0) scale_out[bi * kb + bj] = recip_rn(s);
  uint2* dst = reinterpret_cast<uint2*>(w8 + off);
  uint32_t sat = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) dst[v] = cast8<FMT, HW>(b[v], mx[v], s, sat);
}

// ------------------------------------------------------------------ diagnostics
// Vectors of 8 inputs, decided like the fused kernel: the hardware path unless
// the vector's largest magnitude is NaN or could saturate.
template <int TARGET, bool HW>
__global__ __launch_bounds__(kThreads) void k_convert(const float* __restrict__ x, int64_t n,
                                                      void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t nv = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nv; i += stride) {
    const float4 a = reinterpret_cast<const float4*>(x)[2 * i];
    const float4 c = reinterpret_cast<const float4*>(x)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t m = __float_as_uint(v[j]) & 0x7FFFFFFFu;
      amax = m > amax ? m : amax;
    }
    if constexpr (TARGET == 0 || TARGET == 1) {
      const bool risky = (TARGET == 0) ? (amax > kE4M3SatAbove) : (amax >= kE5M2SatFrom);
      uint2 q;
      if (!HW || risky) {
        q.x = pack4_int<TARGET>(v[0], v[1], v[2], v[3]);
        q.y = pack4_int<TARGET>(v[4], v[5], v[6], v[7]);
      } else {
        q.x = pack4_hw<TARGET>(v[0], v[1], v[2], v[3]);
        q.y = pack4_hw<TARGET>(v[4], v[5], v[6], v[7]);
      }
      reinterpret_cast<uint2*>(out)[i] = q;
    } else if constexpr (TARGET == 2) {
      uint4 r;
      if (!HW || amax > kF32Inf) {
        r = make_uint4(pack2_bf16_int(v[0], v[1]), pack2_bf16_int(v[2], v[3]),
                       pack2_bf16_int(v[4], v[5]), pack2_bf16_int(v[6], v[7]));
      } else {
        r = make_uint4(pack2_bf16_hw(v[0], v[1]), pack2_bf16_hw(v[2], v[3]),
                       pack2_bf16_hw(v[4], v[5]), pack2_bf16_hw(v[6], v[7]));
      }
      reinterpret_cast<uint4*>(out)[i] = r;
    } else if constexpr (TARGET == 5) {
      float r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = __builtin_sqrtf(v[j]);
      reinterpret_cast<float4*>(out)[2 * i] = make_float4(r[0], r[1], r[2], r[3]);
      reinterpret_cast<float4*>(out)[2 * i + 1] = make_float4(r[4], r[5], r[6], r[7]);
    } else {
      uint2 q = make_uint2(0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q.x |= (TARGET == 3 ? saturates<0>(v[j]) : saturates<1>(v[j])) << (8 * j);
        q.y |= (TARGET == 3 ? saturates<0>(v[4 + j]) : saturates<1>(v[4 + j])) << (8 * j);
      }
      reinterpret_cast<uint2*>(out)[i] = q;
    }
  }
}

__global__ void k_scale_rule(const float* __restrict__ amax, int64_t n, float margin, float fmax,
                             float* __restrict__ scale, float* __restrict__ scale_inv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float s = scale_rule(amax[i], margin, fmax);
    scale[i] = s;
    if (scale_inv) scale_inv[i] = recip_rn(s);
  }
}

__global__ __launch_bounds__(kThreads) void k_copy(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < n16; i += 2 * stride) {
    const uint4 a = load_nt(src + i), b = load_nt(src + i + stride);
    store_nt(dst + i, a.x, a.y, a.z, a.w);
    store_nt(dst + i + stride, b.x, b.y, b.z, b.w);
  }
  if (i < n16) {
    const uint4 a = load_nt(src + i);
    store_nt(dst + i, a.x, a.y, a.z, a.w);
  }
}

// ------------------------------------------------------------------ dispatch
template <int FMT, int ACT, bool WBF16, bool AMAX, bool CAST, bool UPD = false>
static int launch_tensor(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout,
                         const float* scale_ptr, fp8dp_acc_slot* slots, hipStream_t stream,
                         fp8dp_tensor_state* st = nullptr) {
  const int64_t n8 = n / 8;
  const int tail = (int)(n % 8);
  const LaunchShape ls = launch_shape(n8, kThreads, WBF16, kBlocksPerCURead);
  const unsigned grid = ls.form == kFormLoop || codec() != 0
                            ? grid_for(n8 > 0 ? n8 : 1, kThreads, WBF16 ? kBlocksPerCU : kBlocksPerCURead)
                            : ls.grid;
#define FP8DP_LAUNCH_T(F)                                                                     \
  hipLaunchKernelGGL((k_quant_tensor<FMT, ACT, WBF16, AMAX, CAST, true, F, UPD>), dim3(grid), \
                     dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(h),            \
                     reinterpret_cast<uint4*>(bout), reinterpret_cast<uint2*>(qout), n8, tail, \
                     scale_ptr, slots, st)
  if (codec() == 0 && ls.form == kFormOne)
    FP8DP_LAUNCH_T(kFormOne);
  else if (codec() == 0 && ls.form == kFormPair)
    FP8DP_LAUNCH_T(kFormPair);
  else if (codec() == 0)
    FP8DP_LAUNCH_T(kFormLoop);
  else
    hipLaunchKernelGGL((k_quant_tensor<FMT, ACT, WBF16, AMAX, CAST, false, kFormLoop, UPD>),
                       dim3(grid), dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(h),
                       reinterpret_cast<uint4*>(bout), reinterpret_cast<uint2*>(qout), n8, tail,
                       scale_ptr, slots, st);
#undef FP8DP_LAUNCH_T
  return check_launch("quantize");
}

// quantize_fused_update: the same launches with the step's end in the last workgroup
template <int FMT, int ACT>
static int dispatch_tensor_update(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout,
                                  fp8dp_tensor_state* st, hipStream_t stream) {
  const float* sp = &st->scale;
  if (bout && qout)
    return launch_tensor<FMT, ACT, true, true, true, true>(h, n, bout, qout, sp, st->acc, stream, st);
  if (bout)
    return launch_tensor<FMT, ACT, true, true, false, true>(h, n, bout, qout, sp, st->acc, stream, st);
  if (qout)
    return launch_tensor<FMT, ACT, false, true, true, true>(h, n, bout, qout, sp, st->acc, stream, st);
  return launch_tensor<FMT, ACT, false, true, false, true>(h, n, bout, qout, sp, st->acc, stream, st);
}

template <int FMT, int ACT>
static int dispatch_tensor(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout,
                           const float* scale_ptr, fp8dp_acc_slot* slots, hipStream_t stream) {
  if (bout && qout)
    return launch_tensor<FMT, ACT, true, true, true>(h, n, bout, qout, scale_ptr, slots, stream);
  if (bout)
    return launch_tensor<FMT, ACT, true, true, false>(h, n, bout, qout, scale_ptr, slots, stream);
  if (qout)
    return launch_tensor<FMT, ACT, false, true, true>(h, n, bout, qout, scale_ptr, slots, stream);
  return launch_tensor<FMT, ACT, false, true, false>(h, n, bout, qout, scale_ptr, slots, stream);
}

template <int FMT, int ACT, bool WBF16, bool WFP8, bool ACC>
static int launch_group(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout, float* gsi,
                        fp8dp_acc_slot* slots, hipStream_t stream) {
  const int64_t n8 = n / 8;
  const LaunchShape ls = launch_shape(n8, kThreads, WBF16, kBlocksPerCURead);
  const unsigned grid = ls.form == kFormLoop || codec() != 0
                            ? grid_for(n8, kThreads, WBF16 ? kBlocksPerCU : kBlocksPerCURead)
                            : ls.grid;
#define FP8DP_LAUNCH_G(F)                                                                      \
  hipLaunchKernelGGL((k_quant_group<FMT, ACT, WBF16, WFP8, ACC, true, F>), dim3(grid),         \
                     dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(h),             \
                     reinterpret_cast<uint4*>(bout), reinterpret_cast<uint2*>(qout), gsi, n8, slots)
  if (codec() == 0 && ls.form == kFormOne)
    FP8DP_LAUNCH_G(kFormOne);
  else if (codec() == 0 && ls.form == kFormPair)
    FP8DP_LAUNCH_G(kFormPair);
  else if (codec() == 0)
    FP8DP_LAUNCH_G(kFormLoop);
  else
    hipLaunchKernelGGL((k_quant_group<FMT, ACT, WBF16, WFP8, ACC, false>), dim3(grid),
                       dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(h),
                       reinterpret_cast<uint4*>(bout), reinterpret_cast<uint2*>(qout), gsi, n8,
                       slots);
#undef FP8DP_LAUNCH_G
  return check_launch("quantize_fused(group)");
}

template <int FMT, int ACT>
static int dispatch_group(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout, float* gsi,
                          fp8dp_acc_slot* slots, hipStream_t stream) {
  const bool acc = slots != nullptr;
#define FP8DP_GROUP_CASE(WB, WQ, AC)                                                       \
  if ((bout != nullptr) == WB && (qout != nullptr) == WQ && acc == AC)                     \
    return launch_group<FMT, ACT, WB, WQ, AC>(h, n, bout, qout, gsi, slots, stream);
  FP8DP_GROUP_CASE(true, true, true)
  FP8DP_GROUP_CASE(true, true, false)
  FP8DP_GROUP_CASE(false, true, true)
  FP8DP_GROUP_CASE(false, true, false)
  FP8DP_GROUP_CASE(true, false, true)
  FP8DP_GROUP_CASE(true, false, false)
  FP8DP_GROUP_CASE(false, false, true)
  FP8DP_GROUP_CASE(false, false, false)
#undef FP8DP_GROUP_CASE
  return FP8DP_EINVAL;
}

template <int FMT, int ACT, bool WBF16>
static int launch_mx_quant(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout,
                           uint8_t* e8, hipStream_t stream) {
  const int64_t n8 = n / 8;
  const LaunchShape ls = launch_shape(n8, kThreads, WBF16, kBlocksPerCURead);
  const unsigned grid = ls.form == kFormLoop || codec() != 0
                            ? grid_for(n8, kThreads, WBF16 ? kBlocksPerCU : kBlocksPerCURead)
                            : ls.grid;
#define FP8DP_LAUNCH_M(F)                                                                   \
  hipLaunchKernelGGL((k_quant_mx<FMT, ACT, WBF16, true, F>), dim3(grid), dim3(kThreads), 0, \
                     stream, reinterpret_cast<const uint4*>(h), reinterpret_cast<uint4*>(bout), \
                     reinterpret_cast<uint2*>(qout), e8, n8)
  if (codec() == 0 && ls.form == kFormOne)
    FP8DP_LAUNCH_M(kFormOne);
  else if (codec() == 0 && ls.form == kFormPair)
    FP8DP_LAUNCH_M(kFormPair);
  else if (codec() == 0)
    FP8DP_LAUNCH_M(kFormLoop);
  else
    hipLaunchKernelGGL((k_quant_mx<FMT, ACT, WBF16, false>), dim3(grid), dim3(kThreads), 0,
                       stream, reinterpret_cast<const uint4*>(h), reinterpret_cast<uint4*>(bout),
                       reinterpret_cast<uint2*>(qout), e8, n8);
#undef FP8DP_LAUNCH_M
  return check_launch("quantize_mx");
}

template <int FMT, int ACT>
static int dispatch_mx(const uint16_t* h, int64_t n, uint16_t* bout, uint8_t* qout, uint8_t* e8,
                       hipStream_t stream) {
  return bout ? launch_mx_quant<FMT, ACT, true>(h, n, bout, qout, e8, stream)
              : launch_mx_quant<FMT, ACT, false>(h, n, bout, qout, e8, stream);
}

template <int FMT, int ACT>
static int launch_recast(const uint16_t* h, int64_t n, uint8_t* qout,
                         const fp8dp_tensor_state* st, hipStream_t stream) {
  const int64_t n8 = n / 8;
  const int tail = (int)(n % 8);
  // a small grid: in the usual case (no overflow) every workgroup only reads
  // the flag, and the launch's cost grows with its workgroup count
  const unsigned grid = grid_for(n8 > 0 ? n8 : 1, kThreads, 2);
  if (codec() == 0)
    hipLaunchKernelGGL((k_quant_recast<FMT, ACT, true>), dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(h), reinterpret_cast<uint2*>(qout), n8,
                       tail, st);
  else
    hipLaunchKernelGGL((k_quant_recast<FMT, ACT, false>), dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(h), reinterpret_cast<uint2*>(qout), n8,
                       tail, st);
  return check_launch("quantize_recompute");
}

static bool valid_fmt(int f) { return f == FP8DP_E4M3 || f == FP8DP_E5M2; }
static bool valid_act(int a) { return a == FP8DP_ACT_IDENTITY || a == FP8DP_ACT_RELU2; }

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int64_t fp8dp_state_size(void) { return (int64_t)sizeof(fp8dp_tensor_state); }

extern "C" int fp8dp_state_init(fp8dp_tensor_state* st, fp8dp_format fmt, int32_t hist_len,
                                float margin, float initial_amax, hipStream_t stream) {
  if (st == nullptr || !aligned16(st)) {
    set_error("fp8dp_state_init: state pointer is NULL or not 16-byte aligned");
    return FP8DP_EINVAL;
  }
  if (!valid_fmt(fmt)) {
    set_error("fp8dp_state_init: unknown format %d", (int)fmt);
    return FP8DP_EINVAL;
  }
  if (hist_len < 1 || hist_len > FP8DP_MAX_HIST) {
    set_error("fp8dp_state_init: hist_len %d outside 1..%d", hist_len, FP8DP_MAX_HIST);
    return FP8DP_EINVAL;
  }
  if (!(margin > 0.0f) || !(margin < 3.4e38f)) {
    set_error("fp8dp_state_init: margin must be a positive finite number");
    return FP8DP_EINVAL;
  }
  hipLaunchKernelGGL(k_state_init, dim3(1), dim3(64), 0, stream, st, (int)fmt, hist_len, margin,
                     initial_amax);
  return check_launch("fp8dp_state_init");
}

extern "C" int amax_history_update(fp8dp_tensor_state* st, hipStream_t stream) {
  if (st == nullptr || !aligned16(st)) {
    set_error("amax_history_update: state pointer is NULL or not 16-byte aligned");
    return FP8DP_EINVAL;
  }
  hipLaunchKernelGGL(k_history_update, dim3(1), dim3(64), 0, stream, st);
  return check_launch("amax_history_update");
}

extern "C" int quantize_fused(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                              fp8dp_format fmt, fp8dp_scale_mode mode, fp8dp_tensor_state* st,
                              uint16_t* bf16_out, uint8_t* fp8_out, float* group_scale_inv,
                              hipStream_t stream) {
  if (h == nullptr || rows < 1 || cols < 1) {
    set_error("quantize_fused: need a non-NULL input and rows, cols >= 1");
    return FP8DP_EINVAL;
  }
  if (!valid_fmt(fmt) || !valid_act(act)) {
    set_error("quantize_fused: unknown format %d or activation %d", (int)fmt, (int)act);
    return FP8DP_EINVAL;
  }
  if (!aligned16(h) || !aligned16(bf16_out) || !aligned16(fp8_out) || !aligned16(st)) {
    set_error("quantize_fused: tensor and state pointers must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  const int64_t n = rows * cols;
  if (mode == FP8DP_PER_TENSOR) {
    if (st == nullptr) {
      set_error("quantize_fused: PER_TENSOR mode needs the scaling state");
      return FP8DP_EINVAL;
    }
    const float* sp = &st->scale;
    fp8dp_acc_slot* slots = st->acc;
    if (fmt == FP8DP_E4M3)
      return act == FP8DP_ACT_RELU2
                 ? dispatch_tensor<0, 1>(h, n, bf16_out, fp8_out, sp, slots, stream)
                 : dispatch_tensor<0, 0>(h, n, bf16_out, fp8_out, sp, slots, stream);
    return act == FP8DP_ACT_RELU2 ? dispatch_tensor<1, 1>(h, n, bf16_out, fp8_out, sp, slots, stream)
                                  : dispatch_tensor<1, 0>(h, n, bf16_out, fp8_out, sp, slots, stream);
  }
  if (mode != FP8DP_PER_GROUP128) {
    set_error("quantize_fused: unknown scale mode %d", (int)mode);
    return FP8DP_EINVAL;
  }
  if (cols % 128 != 0) {
    set_error("quantize_fused: PER_GROUP128 needs cols %% 128 == 0 (cols = %lld)", (long long)cols);
    return FP8DP_EINVAL;
  }
  if (fp8_out != nullptr && group_scale_inv == nullptr) {
    set_error("quantize_fused: PER_GROUP128 with an FP8 output needs group_scale_inv");
    return FP8DP_EINVAL;
  }
  fp8dp_acc_slot* slots = st ? st->acc : nullptr;
  if (fmt == FP8DP_E4M3)
    return act == FP8DP_ACT_RELU2
               ? dispatch_group<0, 1>(h, n, bf16_out, fp8_out, group_scale_inv, slots, stream)
               : dispatch_group<0, 0>(h, n, bf16_out, fp8_out, group_scale_inv, slots, stream);
  return act == FP8DP_ACT_RELU2
             ? dispatch_group<1, 1>(h, n, bf16_out, fp8_out, group_scale_inv, slots, stream)
             : dispatch_group<1, 0>(h, n, bf16_out, fp8_out, group_scale_inv, slots, stream);
}

extern "C" int quantize_fused_update(const uint16_t* h, int64_t rows, int64_t cols,
                                     fp8dp_act act, fp8dp_format fmt, fp8dp_tensor_state* st,
                                     uint16_t* bf16_out, uint8_t* fp8_out, hipStream_t stream) {
  if (h == nullptr || st == nullptr || rows < 1 || cols < 1) {
    set_error("quantize_fused_update: need non-NULL input and state, rows, cols >= 1");
    return FP8DP_EINVAL;
  }
  if (!valid_fmt(fmt) || !valid_act(act)) {
    set_error("quantize_fused_update: unknown format %d or activation %d", (int)fmt, (int)act);
    return FP8DP_EINVAL;
  }
  if (!aligned16(h) || !aligned16(bf16_out) || !aligned16(fp8_out) || !aligned16(st)) {
    set_error("quantize_fused_update: tensor and state pointers must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  const int64_t n = rows * cols;
  if (fmt == FP8DP_E4M3)
    return act == FP8DP_ACT_RELU2 ? dispatch_tensor_update<0, 1>(h, n, bf16_out, fp8_out, st, stream)
                                  : dispatch_tensor_update<0, 0>(h, n, bf16_out, fp8_out, st, stream);
  return act == FP8DP_ACT_RELU2 ? dispatch_tensor_update<1, 1>(h, n, bf16_out, fp8_out, st, stream)
                                : dispatch_tensor_update<1, 0>(h, n, bf16_out, fp8_out, st, stream);
}

extern "C" int quantize_weight(const uint16_t* w, int64_t N, int64_t K, fp8dp_format fmt,
                               fp8dp_scale_mode mode, uint8_t* w8, float* scale_out,
                               hipStream_t stream) {
  if (w == nullptr || w8 == nullptr || scale_out == nullptr || N < 1 || K < 1) {
    set_error("quantize_weight: NULL pointer or empty shape");
    return FP8DP_EINVAL;
  }
  if (!valid_fmt(fmt) || !aligned16(w) || !aligned16(w8) ||
      (reinterpret_cast<uintptr_t>(scale_out) & 7u)) {
    set_error("quantize_weight: bad format or misaligned pointer");
    return FP8DP_EINVAL;
  }
  const bool hw = codec() == 0;
  if (mode == FP8DP_PER_TENSOR) {
    const int64_t n = N * K;
    const int64_t n8 = n / 8;
    const int tail = (int)(n % 8);
    hipLaunchKernelGGL(k_w_zero, dim3(1), dim3(1), 0, stream, scale_out);
    hipLaunchKernelGGL(k_w_amax, dim3(grid_for(n8 > 0 ? n8 : 1, kThreads, 4)), dim3(kThreads), 0,
                       stream, reinterpret_cast<const uint4*>(w), n8, tail,
                       reinterpret_cast<uint32_t*>(scale_out + 1));
    if (fmt == FP8DP_E4M3) {
      hipLaunchKernelGGL(k_w_final<0>, dim3(1), dim3(1), 0, stream, scale_out);
      return launch_tensor<0, 0, false, false, true>(w, n, nullptr, w8, scale_out + 1, nullptr,
                                                     stream);
    }
    hipLaunchKernelGGL(k_w_final<1>, dim3(1), dim3(1), 0, stream, scale_out);
    return launch_tensor<1, 0, false, false, true>(w, n, nullptr, w8, scale_out + 1, nullptr,
                                                   stream);
  }
  if (mode != FP8DP_PER_GROUP128 || N % 128 != 0 || K % 128 != 0) {
    set_error("quantize_weight: 128 x 128 blocks need N %% 128 == 0 and K %% 128 == 0");
    return FP8DP_EINVAL;
  }
  const unsigned blocks = (unsigned)((N / 128) * (K / 128));
  if (fmt == FP8DP_E4M3) {
    if (hw) hipLaunchKernelGGL((k_w_block<0, true>), dim3(blocks), dim3(kThreads), 0, stream, w, K, w8, scale_out);
    else hipLaunchKernelGGL((k_w_block<0, false>), dim3(blocks), dim3(kThreads), 0, stream, w, K, w8, scale_out);
  } else {
    if (hw) hipLaunchKernelGGL((k_w_block<1, true>), dim3(blocks), dim3(kThreads), 0, stream, w, K, w8, scale_out);
    else hipLaunchKernelGGL((k_w_block<1, false>), dim3(blocks), dim3(kThreads), 0, stream, w, K, w8, scale_out);
  }
  return check_launch("quantize_weight");
}

extern "C" int fp8dp_bench_act_bf16(const uint16_t* h, int64_t n, fp8dp_act act, uint16_t* out,
                                    hipStream_t stream) {
  if (h == nullptr || out == nullptr || n < 1 || !valid_act(act) || !aligned16(h) ||
      !aligned16(out)) {
    set_error("fp8dp_bench_act_bf16: bad arguments");
    return FP8DP_EINVAL;
  }
  return act == FP8DP_ACT_RELU2
             ? launch_tensor<0, 1, true, false, false>(h, n, out, nullptr, nullptr, nullptr, stream)
             : launch_tensor<0, 0, true, false, false>(h, n, out, nullptr, nullptr, nullptr, stream);
}

extern "C" int fp8dp_bench_amax(const uint16_t* x, int64_t n, fp8dp_tensor_state* st,
                                hipStream_t stream) {
  if (x == nullptr || st == nullptr || n < 1 || !aligned16(x) || !aligned16(st)) {
    set_error("fp8dp_bench_amax: bad arguments");
    return FP8DP_EINVAL;
  }
  return launch_tensor<0, 0, false, true, false>(x, n, nullptr, nullptr, nullptr, st->acc, stream);
}

extern "C" int fp8dp_bench_cast(const uint16_t* x, int64_t n, fp8dp_format fmt,
                                fp8dp_tensor_state* st, uint8_t* out, hipStream_t stream) {
  if (x == nullptr || st == nullptr || out == nullptr || n < 1 || !valid_fmt(fmt) ||
      !aligned16(x) || !aligned16(st) || !aligned16(out)) {
    set_error("fp8dp_bench_cast: bad arguments");
    return FP8DP_EINVAL;
  }
  if (fmt == FP8DP_E4M3)
    return launch_tensor<0, 0, false, false, true>(x, n, nullptr, out, &st->scale, st->acc, stream);
  return launch_tensor<1, 0, false, false, true>(x, n, nullptr, out, &st->scale, st->acc, stream);
}

extern "C" int fp8dp_bench_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes < 16 || bytes % 16 || !aligned16(src) ||
      !aligned16(dst)) {
    set_error("fp8dp_bench_copy: bad arguments");
    return FP8DP_EINVAL;
  }
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_copy, dim3(grid_for(n16, kThreads, kBlocksPerCU)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n16);
  return check_launch("fp8dp_bench_copy");
}

extern "C" int fp8dp_convert_f32(const float* x, int64_t n, int32_t target, void* out,
                                 hipStream_t stream) {
  if (x == nullptr || out == nullptr || n < 8 || n % 8 || target < 0 || target > 5 ||
      !aligned16(x) || !aligned16(out)) {
    set_error("fp8dp_convert_f32: bad arguments (n must be a positive multiple of 8)");
    return FP8DP_EINVAL;
  }
  const unsigned grid = grid_for(n / 8, kThreads, 8);
  const bool hw = codec() == 0;
#define FP8DP_CONV(T)                                                                           \
  if (target == T) {                                                                            \
    if (hw) hipLaunchKernelGGL((k_convert<T, true>), dim3(grid), dim3(kThreads), 0, stream, x, n, out); \
    else hipLaunchKernelGGL((k_convert<T, false>), dim3(grid), dim3(kThreads), 0, stream, x, n, out); \
  }
  FP8DP_CONV(0)
  FP8DP_CONV(1)
  FP8DP_CONV(2)
  FP8DP_CONV(3)
  FP8DP_CONV(4)
  FP8DP_CONV(5)
#undef FP8DP_CONV
  return check_launch("fp8dp_convert_f32");
}

extern "C" int fp8dp_scale_rule(const float* amax, int64_t n, float margin, fp8dp_format fmt,
                                float* scale, float* scale_inv, hipStream_t stream) {
  if (amax == nullptr || scale == nullptr || n < 1 || !valid_fmt(fmt)) {
    set_error("fp8dp_scale_rule: bad arguments");
    return FP8DP_EINVAL;
  }
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_scale_rule, dim3(grid), dim3(256), 0, stream, amax, n, margin,
                     fmt == FP8DP_E4M3 ? 448.0f : 57344.0f, scale, scale_inv);
  return check_launch("fp8dp_scale_rule");
}

extern "C" int quantize_mx(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                           fp8dp_format fmt, uint16_t* bf16_out, uint8_t* fp8_out,
                           uint8_t* scale_out, hipStream_t stream) {
  if (h == nullptr || fp8_out == nullptr || scale_out == nullptr) {
    set_error("quantize_mx: NULL input, code or exponent pointer");
    return FP8DP_EINVAL;
  }
  if (rows < 1 || cols < 32 || cols % 32 != 0) {
    set_error("quantize_mx: need rows >= 1 and cols a positive multiple of 32 (got %lld, %lld)",
              (long long)rows, (long long)cols);
    return FP8DP_EINVAL;
  }
  if (!valid_fmt(fmt) || !valid_act(act)) {
    set_error("quantize_mx: unknown format %d or activation %d", (int)fmt, (int)act);
    return FP8DP_EINVAL;
  }
  if (!aligned16(h) || !aligned16(bf16_out) || !aligned16(fp8_out)) {
    set_error("quantize_mx: input, copy and code pointers must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  const int64_t n = rows * cols;
  if (fmt == FP8DP_E4M3)
    return act == FP8DP_ACT_RELU2 ? dispatch_mx<0, 1>(h, n, bf16_out, fp8_out, scale_out, stream)
                                  : dispatch_mx<0, 0>(h, n, bf16_out, fp8_out, scale_out, stream);
  return act == FP8DP_ACT_RELU2 ? dispatch_mx<1, 1>(h, n, bf16_out, fp8_out, scale_out, stream)
                                : dispatch_mx<1, 0>(h, n, bf16_out, fp8_out, scale_out, stream);
}

extern "C" int quantize_recompute(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                                  fp8dp_format fmt, const fp8dp_tensor_state* st,
                                  uint8_t* fp8_out, hipStream_t stream) {
  if (h == nullptr || st == nullptr || fp8_out == nullptr || rows < 1 || cols < 1) {
    set_error("quantize_recompute: need non-NULL h, st, fp8_out and rows, cols >= 1");
    return FP8DP_EINVAL;
  }
  if (!valid_fmt(fmt) || !valid_act(act)) {
    set_error("quantize_recompute: unknown format %d or activation %d", (int)fmt, (int)act);
    return FP8DP_EINVAL;
  }
  if (!aligned16(h) || !aligned16(fp8_out) || !aligned16(st)) {
    set_error("quantize_recompute: tensor and state pointers must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  const int64_t n = rows * cols;
  if (fmt == FP8DP_E4M3)
    return act == FP8DP_ACT_RELU2 ? launch_recast<0, 1>(h, n, fp8_out, st, stream)
                                  : launch_recast<0, 0>(h, n, fp8_out, st, stream);
  return act == FP8DP_ACT_RELU2 ? launch_recast<1, 1>(h, n, fp8_out, st, stream)
                                : launch_recast<1, 0>(h, n, fp8_out, st, stream);
}
