// w4a4_common.hpp — device-side pieces shared by the NVFP4 and MXFP4 kernels:
// vector types, the kernel parameter block, the LDS swizzle, wait/barrier
// helpers, direct-to-LDS DMA, the LoRA MFMA and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace w4a4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const uint8_t* act;
  const uint8_t* ascales;
  const uint8_t* wgt;
  const uint8_t* wscales;
  const float* wcscale;
  const float* bias;
  const uint16_t* lora_act_in;
  const uint16_t* lora_up;
  uint16_t* out;
  int M, N, K, R;
  int tiles_m, tiles_n;   // tile rows and columns of this launch
  int tm0;                // its first tile row (in this instance's BM rows) within the M rows
  float* part;            // a K-sliced launch: fp32 sums, [gridDim.y slices][part_rows][N]
  int part_row0, part_rows;   // the output rows those sums cover
};

// 16-byte chunk c of a 64-byte row is stored at chunk position c ^ swz(row).
// The consumers read one 16-byte chunk of each of 32 consecutive rows per
// half-wave (ds_read_b128). Measured with the LDS bank-conflict counter on
// gfx950: unswizzled rows cost 12 extra cycles per such read, an XOR by row
// bits 1-2 or 1^3,2^4 still 4, and an XOR by row bits 2-3 none.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt vmcnt(VM) lgkmcnt(0), gfx9 encoding (vmcnt split over bits 3:0 and 15:14).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}

// s_waitcnt vmcnt(VM) only (expcnt and lgkmcnt at their maxima: no wait).
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
}

// f.template operator()<I>() for I = I0 .. N-1 in order: an unrolled loop whose
// index is a constant expression in the body, so that register arrays indexed
// by it are resolved before the compiler decides where the arrays live.
template <int I0, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f.template operator()<I0>();
    static_for<I0 + 1, N>(f);
  }
}

// Workgroup barrier without the memory fence __syncthreads() carries: the
// fence would wait for every outstanding DMA (vmcnt(0)) and serialize the
// ring. Each caller waits for exactly the DMA it needs first; the asm memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Direct-to-LDS copy: lane l of the wave writes BYTES bytes at lds_wave_base + l*BYTES.
template <int BYTES>
__device__ __forceinline__ void dma(const void* gsrc, void* lds_wave_base) {
  static_assert(BYTES == 16 || BYTES == 4, "gfx950 DMA piece sizes used here");
  const auto src = (const __attribute__((address_space(1))) void*)gsrc;
  const auto dst = (__attribute__((address_space(3))) void*)lds_wave_base;
  if constexpr (BYTES == 16) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
  } else {
    __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
  }
}

// One LoRA k-step: 8 ranks per lane of lora_up (rows n) and lora_act_in
// (rows m) as raw 16-bit patterns, fp16 or bf16; both MFMAs have the K-loop's
// 32x32 accumulator layout.
template <bool F16>
__device__ __forceinline__ f32x16 lora_mfma(u32x4 up, u32x4 act, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, up), __builtin_bit_cast(f16x8, act),
                                                  c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, up), __builtin_bit_cast(bf16x8, act),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_pair(uint16_t lo, uint16_t hi) {
  return uint32_t(lo) | (uint32_t(hi) << 16);
}

// Tile order: workgroups are dealt round-robin to the 8 XCDs (workgroup b
// runs on XCD b % 8), each with its own L2. Renumber so that each XCD gets a
// contiguous run of tiles, and walk that run GROUP tile-rows at a time, so
// the A rows and B columns one XCD reads concurrently stay in its L2.
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcd = 8, kGroup = 4;
  const int T = tiles_m * tiles_n;
  const int per = T / kXcd, rem = T % kXcd;
  const int x = b % kXcd, l = b / kXcd;
  const int L = x < rem ? x * (per + 1) + l : rem * (per + 1) + (x - rem) * per + l;
  const int span = kGroup * tiles_n;
  const int first = (L / span) * kGroup;
  const int gsz = min(tiles_m - first, kGroup);
  const int in = L % span;
  tm = first + in % gsz;
  tn = in / gsz;
}

}  // namespace w4a4
