// gemm_core.hpp -- pieces shared by the matrix kernels (gfx950): MFMA
// operand types, the LDS tile layout, the workgroup -> tile order, direct
// global -> LDS copies and the barrier / wait primitives of the pipelined
// large-tile loop.
#pragma once
#include <hip/hip_runtime.h>

#include <utility>
#include <stdint.h>

namespace fp8dp {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;   // bytes of K per LDS stage (one 128-byte row per operand row)

// LDS layout of a tile with 128-byte rows: 16-byte chunk c of row r sits at
// chunk c ^ ((r / 2) % 8).  gfx950's LDS serves 16 lanes of a 16-byte read
// per cycle from 64 banks (256 bytes, two rows); a fragment read has those 16
// lanes on 16 consecutive rows at one logical chunk, and (r % 2, (r / 2) % 8)
// takes all 16 values over them, so the 16 chunks hit 16 distinct bank groups.
// (The 32-bank pattern c ^ (r % 8) gives rows r and r + 8 the same banks.)
__device__ __forceinline__ int swz(int r, int chunk) {
  return r * kBK + ((chunk ^ ((r >> 1) & 7)) << 4);
}

// blockIdx -> output tile.  Workgroups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8); renumbering so that each XCD receives a
// contiguous run of tiles keeps tiles that share A rows in one XCD's L2.
__device__ __forceinline__ int tile_of_block(int b, int ntiles) {
  const int per = ntiles / 8;
  if (per * 8 != ntiles) return b;
  return (b % 8) * per + b / 8;
}

// Persistent grids: G workgroups walk ntiles tiles.  With ntiles and G both
// multiples of 8, workgroup b (on XCD b % 8) takes tiles b / 8, b / 8 + G / 8,
// ... of that XCD's contiguous run of ntiles / 8 tiles (pass 0 is exactly
// tile_of_block); otherwise tiles b, b + G, ...  tiles_of_block() is the
// number of passes of workgroup b; tile_of_pass() the tile of pass p.
__device__ __forceinline__ int tiles_of_block(int b, int G, int ntiles) {
  if (ntiles % 8 == 0 && G % 8 == 0) {
    const int per = ntiles / 8, gx = G / 8, l = b / 8;
    return l < per ? (per - l + gx - 1) / gx : 0;
  }
  return b < ntiles ? (ntiles - b + G - 1) / G : 0;
}
__device__ __forceinline__ int tile_of_pass(int b, int p, int G, int ntiles) {
  if (ntiles % 8 == 0 && G % 8 == 0) return (b % 8) * (ntiles / 8) + b / 8 + p * (G / 8);
  return b + p * G;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (compile-time
// indices, for instruction operands that must be constants).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Global -> LDS copies (global_load_lds): lane i's 16 bytes land at l + 16 i,
// l the wave-uniform LDS address in M0.  Issued as inline assembly, with the
// one wait state a write of M0 needs before the copy reads it, so that the
// compiler does not track them: it cannot tell which LDS bytes a copy writes,
// and it would make every LDS access after one (the fragment reads of other
// stages, an epilogue's staging) wait for every copy in flight -- and for
// every store, which shares the same counter.  The kernels wait for their
// copies themselves (wait_vmcnt, then a barrier) before any read of them.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* g, uint8_t* l) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_void_t*)l;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(la) : "memory");
}

// The 4-byte form: lane i's dword lands at l + 4 i.
__device__ __forceinline__ void copy4_to_lds(const uint8_t* g, uint8_t* l) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_void_t*)l;
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "{m0}"(la) : "memory");
}


// s_waitcnt with vmcnt(N) and no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that neither the compiler's scheduler nor its memory
// model may move anything across, and that leaves the memory counters alone
// (__syncthreads() would also drain every copy in flight).
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace fp8dp
