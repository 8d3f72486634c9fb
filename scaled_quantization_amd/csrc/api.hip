// api.hip -- error reporting and process-wide switches of the C ABI.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>

#include "common.hpp"

namespace fp8dp {

static thread_local char g_err[512] = "";
static std::atomic<int32_t> g_grid_limit{0};
static std::atomic<int32_t> g_codec{0};
static std::atomic<int32_t> g_cus[64];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

int32_t grid_limit() { return g_grid_limit.load(std::memory_order_relaxed); }
int32_t codec() { return g_codec.load(std::memory_order_relaxed); }

// Compute units of the current device (cached per device).
int32_t num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int32_t n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  g_cus[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace fp8dp

extern "C" const char* fp8dp_last_error(void) { return fp8dp::g_err; }

extern "C" int32_t fp8dp_set_grid_limit(int32_t blocks) {
  return fp8dp::g_grid_limit.exchange(blocks < 0 ? 0 : blocks);
}

extern "C" int32_t fp8dp_set_codec(int32_t c) {
  return fp8dp::g_codec.exchange(c == 1 ? 1 : 0);
}
