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

}  // namespace fp8dp
