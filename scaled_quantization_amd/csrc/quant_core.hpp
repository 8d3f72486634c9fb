// quant_core.hpp -- the quantizer's per-vector steps, shared by the
// element-wise quantizer and by the GEMM whose epilogue quantizes: squared
// ReLU on BF16 pairs, the largest magnitude of a vector, the scaled
// saturating cast with its saturation count, one-element tails, and the
// block reduction of (amax, count) into the state's accumulator slots.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "fp8dp.h"

namespace fp8dp {

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt_t __attribute__((ext_vector_type(2)));

// 16- and 8-byte loads marked non-temporal (streamed data that is not read again).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  const u32x2_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt_t*>(p));
  return make_uint2(v.x, v.y);
}

// Streaming stores: the outputs are not read again by this kernel, so they
// should not displace the inputs from the caches.
__device__ __forceinline__ void store_nt(uint4* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(u32x4_nt_t{a, b, c, d}, reinterpret_cast<u32x4_nt_t*>(p));
}
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
  __builtin_nontemporal_store(u32x2_nt_t{v.x, v.y}, reinterpret_cast<u32x2_nt_t*>(p));
}

// Largest 16-bit magnitude among the 8 BF16 values of a vector.
template <bool SIGNED>
__device__ __forceinline__ uint32_t vec_absmax16(const uint32_t b[4]) {
  ushort2_t m = {0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = SIGNED ? (b[j] & 0x7FFF7FFFu) : b[j];
    m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, w));
  }
  return m.x > m.y ? m.x : m.y;
}

// BF16 activation of one packed pair (low half first).
template <int ACT, bool HW>
__device__ __forceinline__ uint32_t act_pair(uint32_t w) {
  if constexpr (ACT == FP8DP_ACT_IDENTITY) {
    return w;
  } else {
    const float lo = relu2(__uint_as_float(w << 16));
    const float hi = relu2(__uint_as_float(w & 0xFFFF0000u));
    return HW ? pack2_bf16_hw(lo, hi) : pack2_bf16_int(lo, hi);
  }
}

// Casts the 8 BF16 values of a vector with multiplier s; returns the 8 codes
// packed little-endian and adds saturating elements to `sat`.  `mx` is the
// vector's largest BF16 magnitude.
template <int FMT, bool HW>
__device__ __forceinline__ uint2 cast8(const uint32_t b[4], uint32_t mx, float s, uint32_t& sat) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __fmul_rn(__uint_as_float(b[j] << 16), s);
    v[2 * j + 1] = __fmul_rn(__uint_as_float(b[j] & 0xFFFF0000u), s);
  }
  const uint32_t vmax = __float_as_uint(__fmul_rn(__uint_as_float(mx << 16), s));
  const bool risky = (FMT == 0) ? (vmax > kE4M3SatAbove) : (vmax >= kE5M2SatFrom);
  uint2 q;
  if (!HW || risky) {
    q.x = pack4_int<FMT>(v[0], v[1], v[2], v[3]);
    q.y = pack4_int<FMT>(v[4], v[5], v[6], v[7]);
    if (risky) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sat += saturates<FMT>(v[j]);
    }
  } else {
    q.x = pack4_hw<FMT>(v[0], v[1], v[2], v[3]);
    q.y = pack4_hw<FMT>(v[4], v[5], v[6], v[7]);
  }
  return q;
}

// One element (ragged tails): returns its BF16 copy, code and counts.
template <int FMT, int ACT>
__device__ __forceinline__ void quant_one(uint16_t h, float s, uint16_t& b, uint8_t& q,
                                          uint32_t& amax16, uint32_t& sat) {
  uint32_t bb = h;
  if constexpr (ACT == FP8DP_ACT_RELU2) bb = bf16_rne_int(relu2(__uint_as_float((uint32_t)h << 16)));
  b = (uint16_t)bb;
  const uint32_t mag = bb & 0x7FFFu;
  amax16 = mag > amax16 ? mag : amax16;
  const float v = __fmul_rn(__uint_as_float(bb << 16), s);
  q = (uint8_t)enc_int<FMT>(v);
  sat += saturates<FMT>(v);
}

// ------------------------------------------------------------------ MXFP8
// "FP8 training: what it is and how it works", Trade-offs and edge cases: the
// microscaling recipe scales each block of 32 adjacent values by its own
// power of two.  Block exponent k (decode scale 2^k, stored as the E8M0 byte
// k + 127): the smallest k in [-127, 127] with |b| <= max * 2^k for every
// element of the block.  From the block's largest BF16 magnitude pattern m
// (sign cleared; NaN patterns order above infinity): for a normal m = 1.f 2^e
// and max = 1.75 * 2^emax, k = e - emax, plus one when the fraction exceeds
// 0.75 (7-bit field above 0x60); zero and subnormal BF16 values lie below
// max * 2^-127 (k = -127); infinity and NaN admit no k (k = 127).
template <int FMT>
__device__ __forceinline__ int mx_exponent(uint32_t m) {
  constexpr int emax = FMT == 0 ? 8 : 15;
  const int ef = (int)(m >> 7);
  if (ef >= 0xFF) return 127;
  if (ef == 0) return -127;
  const int k = ef - 127 - emax + ((m & 0x7Fu) > 0x60u ? 1 : 0);
  return k < -127 ? -127 : k;
}

// 2^-k in binary32 (k = 127 gives the subnormal 2^-127).
__device__ __forceinline__ float mx_multiplier(int k) {
  return __uint_as_float(k == 127 ? 0x00400000u : (uint32_t)(127 - k) << 23);
}

// Block-wide reduction of (amax16, sat) and one atomic pair into a slot.
// NT: threads of the block (a multiple of 64); every thread must call it.
// sm: 2 NT / 64 words of LDS scratch.  Kernels that copy global memory
// straight into LDS keep all their LDS in one array and pass a part of it:
// with a second LDS variable the compiler tracks the copies per variable and
// makes every read of the copied array wait for all copies in flight.
template <int NT>
__device__ __forceinline__ void block_fold_in(uint32_t amax16, uint32_t sat,
                                              fp8dp_acc_slot* slots, uint32_t* sm) {
  uint32_t* s_max = sm;
  uint32_t* s_sat = sm + NT / 64;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t om = __shfl_xor(amax16, off);
    amax16 = om > amax16 ? om : amax16;
    sat += __shfl_xor(sat, off);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_max[w] = amax16;
    s_sat[w] = sat;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      m = s_max[i] > m ? s_max[i] : m;
      c += s_sat[i];
    }
    fp8dp_acc_slot* slot = slots + (blockIdx.x % FP8DP_ACC_SLOTS);
    if (m) atomicMax(&slot->amax, m << 16);
    if (c) atomicAdd((unsigned long long*)&slot->sat, (unsigned long long)c);
  }
}

template <int NT>
__device__ __forceinline__ void block_fold(uint32_t amax16, uint32_t sat, fp8dp_acc_slot* slots) {
  __shared__ uint32_t sm[2 * (NT / 64)];
  block_fold_in<NT>(amax16, sat, slots, sm);
}

// Closes a step of delayed scaling; run by one wave (lane l reduces
// accumulator slot l and holds history entry l).  Every load is issued
// before any use; the ring after this step's write -- entry pos replaced by
// the step's amax -- is reduced in registers.  The slots are read with
// device-scope atomic loads: in the fused form other workgroups of the same
// launch wrote them moments before (with atomics, at the device's L2).
__device__ __forceinline__ void state_update_wave(fp8dp_tensor_state* st) {
  const int l = threadIdx.x & 63;
  uint32_t m = __hip_atomic_load(&st->acc[l].amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t c = __hip_atomic_load(&st->acc[l].sat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float h = l < FP8DP_MAX_HIST ? st->history[l] : 0.0f;
  const int len = st->hist_len;
  const int pos = st->hist_pos;
  const float margin = st->margin;
  const int fmt = st->fmt;
  const float sinv = st->scale_inv;
  const uint32_t steps = st->steps;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t om = __shfl_xor(m, off);
    m = om > m ? om : m;
    const uint32_t clo = __shfl_xor((uint32_t)c, off);
    const uint32_t chi = __shfl_xor((uint32_t)(c >> 32), off);
    c += ((uint64_t)chi << 32) | clo;
  }
  const float amax_t = __uint_as_float(m);
  uint32_t hm = l < len ? (__float_as_uint(l == pos ? amax_t : h) & 0x7FFFFFFFu) : 0u;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(hm, off);
    hm = o > hm ? o : hm;
  }
  st->acc[l].amax = 0;
  st->acc[l].sat = 0;
  st->acc[l].ticket = 0;
  if (l == 0) {
    st->history[pos] = amax_t;
    st->hist_pos = (pos + 1 == len) ? 0 : pos + 1;
    st->scale_inv_used = sinv;
    const float s = scale_rule(__uint_as_float(hm), margin, fmt == 0 ? 448.0f : 57344.0f);
    st->scale = s;
    st->scale_inv = recip_rn(s);
    st->sat_last = c;
    st->overflow = c > 0 ? 1u : 0u;
    st->amax_last = amax_t;
    st->steps = steps + 1;
    st->ticket = 0;
  }
}

// The block reduction of block_fold_in, then the step's end in the workgroup
// that folds last.  After the block reduction only wave 0 stays.  Thread 0
// adds its workgroup's (amax, count) to its slot with atomics it waits for
// (so they have been performed at the device's point of coherence), then
// counts the workgroup on the slot's ticket; the workgroup that completes a
// slot -- the slot takes workgroups b with b % 64 == j -- counts the slot on
// st->ticket; the one that completes the last slot runs state_update_wave,
// whose device-scope loads see every slot's final values.  Atomics only, no
// fence: a device-scope release would write back this XCD's L2 in every
// workgroup (measured 22x slower), and the accumulators are never written
// any other way.  No workgroup waits for another.  sm: 2 NT / 64 words of LDS.
template <int NT>
__device__ __forceinline__ void block_fold_update(uint32_t amax16, uint32_t sat,
                                                  fp8dp_tensor_state* st, uint32_t* sm) {
  uint32_t* s_max = sm;
  uint32_t* s_sat = sm + NT / 64;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t om = __shfl_xor(amax16, off);
    amax16 = om > amax16 ? om : amax16;
    sat += __shfl_xor(sat, off);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_max[w] = amax16;
    s_sat[w] = sat;
  }
  __syncthreads();
  // waves 1.. leave here instead of waiting for thread 0's round trips
  if (threadIdx.x >= 64) return;
  uint32_t last = 0;
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      m = s_max[i] > m ? s_max[i] : m;
      c += s_sat[i];
    }
    const uint32_t G = gridDim.x, j = blockIdx.x % FP8DP_ACC_SLOTS;
    fp8dp_acc_slot* slot = st->acc + j;
    // both atomics in flight together; the ticket is issued only once the
    // memory counter shows them performed (vmcnt counts atomics and stores)
    if (m) __hip_atomic_fetch_max(&slot->amax, m << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c) __hip_atomic_fetch_add(&slot->sat, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
    const uint32_t nj = G / FP8DP_ACC_SLOTS + (j < G % FP8DP_ACC_SLOTS ? 1u : 0u);
    const uint32_t nslots = G < FP8DP_ACC_SLOTS ? G : FP8DP_ACC_SLOTS;
    if (__hip_atomic_fetch_add(&slot->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        nj - 1)
      last = __hip_atomic_fetch_add(&st->ticket, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == nslots - 1 ? 1u : 0u;
  }
  if (__shfl(last, 0)) state_update_wave(st);
}

}  // namespace fp8dp
