// common.hpp -- host-side helpers shared by the library's translation units:
// error reporting across the C ABI, argument checks and launch settings.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>

#include "fp8dp.h"

namespace fp8dp {

// Records the message returned by fp8dp_last_error() for this thread.
void set_error(const char* fmt, ...);
void clear_error();

// Process-wide scheduling switches (see fp8dp_set_grid_limit / fp8dp_set_codec).
int32_t grid_limit();
int32_t codec();
int32_t num_cus();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Returns FP8DP_EHIP with a message if the last launch failed.
inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return FP8DP_EHIP;
  }
  clear_error();
  return FP8DP_OK;
}

// Thread-block count for a grid-stride element-wise kernel covering `work`
// items of blockDim threads each: enough blocks to fill every compute unit
// several times over, never more than the work needs.
inline unsigned grid_for(int64_t work_items, int block_threads, int blocks_per_cu) {
  int64_t need = (work_items + block_threads - 1) / block_threads;
  int64_t cap = (int64_t)num_cus() * blocks_per_cu;
  if (cap > ((int64_t)1 << 30)) cap = (int64_t)1 << 30;   // grid-stride loops cover the rest
  int32_t lim = grid_limit();
  if (lim > 0 && cap > lim) cap = lim;
  if (need > cap) need = cap;
  if (need < 1) need = 1;
  return (unsigned)need;
}

// Launch forms of the element-wise kernels over n8 8-element vectors:
//   kFormOne  -- a thread per vector, no loop (kernels that write at least as
//                many bytes as they read, and small read-heavy launches);
//   kFormPair -- two vectors per thread, vectors b*2T + t and b*2T + T + t of
//                block b (T threads), both loaded first, no loop (kernels that
//                read more than they write, from kPairMinVectors vectors on);
//   kFormLoop -- grid-stride loop over a capped grid, where the grid of the
//                other forms would exceed the grid cap or a set grid limit.
// Measured at the GPT-2 shape and on a 512 MiB gradient (E5M2 cast):
// one vector per thread is 5% faster than two for the quantizer with its BF16
// copy; for the cast without it two per thread match the loop at 96 MiB and
// beat it by 30% at 512 MiB (6.56 vs 5.03 TB/s); one per thread is 7-22% slower
// than the loop there.  Below about 2^21 vectors one per thread wins for
// read-heavy kernels too (E5M2 cast of a [16384 x 768] gradient, 1.6 M
// vectors: 9.12 us against 9.52 with two; at [65536 x 4096] two win, 124.1
// against 134.7 us; at 6.3 M vectors the cast without the BF16 copy ties).
enum : int { kFormLoop = 0, kFormOne = 1, kFormPair = 2 };
constexpr int64_t kPairMinVectors = (int64_t)1 << 21;
struct LaunchShape {
  unsigned grid;
  int form;
};
inline LaunchShape launch_shape(int64_t n8, int block_threads, bool write_heavy,
                                int loop_blocks_per_cu) {
  const int per = write_heavy || n8 < kPairMinVectors ? 1 : 2;
  int64_t need = (n8 + (int64_t)per * block_threads - 1) / ((int64_t)per * block_threads);
  if (need < 1) need = 1;
  const unsigned g = grid_for(need * block_threads, block_threads, 1 << 20);
  if ((int64_t)g == need) return {g, per == 1 ? kFormOne : kFormPair};
  return {grid_for(n8 > 0 ? n8 : 1, block_threads, loop_blocks_per_cu), kFormLoop};
}

}  // namespace fp8dp
