// mfma_peak.hip — attainable MFMA peak on this chip: one workgroup of four
// waves per compute unit, every wave issuing back-to-back MFMAs of one kind
// into eight independent accumulators (enough to keep the matrix pipe busy
// without a dependent stall), nothing else. Its rate is the ceiling the GEMM
// kernels' MFMA instructions can reach under full-chip load, clock and power
// limits included; the published dense peaks assume the maximum engine clock.
// Each workgroup also records its shader-clock cycles (s_memtime) and
// wall-clock ticks (s_memrealtime, 100 MHz) so the host can report the clock
// the chip actually ran at.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "w4a4_probes.h"
#include "w4a4_common.hpp"
#include "w4a4_host.hpp"
#include "w4a4_layout.hpp"

namespace w4a4 {

constexpr int kPeakThreads = 256;
constexpr int kPeakChains = 8;

template <int KIND>
__global__ __launch_bounds__(kPeakThreads, 1) void mfma_peak_kernel(int iters, uint64_t* clocks) {
  const int tid = threadIdx.x;
  const uint32_t seed = 0x3c003c00u ^ uint32_t(tid * 0x9e3779b9u);
  f32x16 acc[kPeakChains];
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  const u32x4 a = {seed & 0x3fff3fffu, 0x3c003c00u, seed & 0x37ff37ffu, 0x3c003c00u};
  const u32x4 b = {0x3c003c00u, seed & 0x3bff3bffu, 0x3c003c00u, seed & 0x33ff33ffu};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) {
      if constexpr (KIND == 0) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                        acc[c], 0, 0, 0);
      } else if constexpr (KIND == 1) {
        typedef int v8i __attribute__((ext_vector_type(8)));
        const v8i av = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
        const v8i bv = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[c], 4, 4, 0, 127, 0, 127);
      } else {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), acc[c], 0, 0, 0);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  if (tid == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    // keeps the MFMAs alive: a sum equal to this value does not occur
    clocks[2 * blockIdx.x + 1] = (sum == 1.2345e-30f) ? 0 : r1 - r0;
  }
}

}  // namespace w4a4

using namespace w4a4;

extern "C" int w4a4_probe_mfma_peak(int kind, int iters, uint64_t* clocks, void* stream) {
  if (kind < 0 || kind > 2 || iters < 1 || !clocks) return GEMM_W4A4_EINVAL;
  if (reinterpret_cast<uintptr_t>(clocks) & 7u) return GEMM_W4A4_EALIGN;
  const int dev_rc = check_device();
  if (dev_rc != GEMM_W4A4_OK) return dev_rc;
  void (*k)(int, uint64_t*) = kind == 0 ? mfma_peak_kernel<0> : kind == 1 ? mfma_peak_kernel<1> : mfma_peak_kernel<2>;
  void* args[] = {&iters, &clocks};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k), dim3(W4A4_PROBE_GROUPS),
                                       dim3(kPeakThreads), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}
