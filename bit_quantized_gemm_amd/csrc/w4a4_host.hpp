// w4a4_host.hpp — host-side checks shared by the library's entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "gemm_w4a4.h"

namespace w4a4 {

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = uintptr_t(a), y = uintptr_t(b);
  return x < y + nb && y < x + na;
}

inline std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, 2 other

inline int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_W4A4_EDEVICE;
  if (dev < 0 || dev >= 64) return GEMM_W4A4_EDEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_W4A4_EDEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? GEMM_W4A4_OK : GEMM_W4A4_EDEVICE;
}

}  // namespace w4a4
