// w4a4_host.hpp — host side shared by the library's entry points: argument
// checks, the compiled-instance descriptor, the launch plan (budget, rounds,
// registers) and the launch itself.
#pragma once

#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "gemm_w4a4.h"
#include "w4a4_common.hpp"
#include "w4a4_layout.hpp"
#include "w4a4_resources.h"

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

// Resource figures of a kernel from the table the build generated out of the
// code objects: the kernel handle's symbol (dladdr) names its table row.
inline const KernelResources* find_resources(const void* kernel) {
  Dl_info info;
  if (!kernel || !dladdr(kernel, &info) || !info.dli_sname) return nullptr;
  for (int i = 0; i < kNumKernelResources; ++i)
    if (strcmp(kKernelResources[i].symbol, info.dli_sname) == 0) return &kKernelResources[i];
  return nullptr;
}

// One compiled tile instance of a kernel family.
struct VariantDesc {
  const void* kernel[2][3];   // [F16][flavour: general, fast, fast with act-scale windows]
  bool has_window;            // the third flavour exists
  int block_m, block_n, block_k, waves_m, waves_n, k_groups, threads, occ, stage_bytes, policy;
  Budget budget;
  double cost;                // time per output element of a full round, relative to 256x192
};

template <class C>
VariantDesc describe(const void* const (&k)[2][3], bool has_window, double cost) {
  return VariantDesc{{{k[0][0], k[0][1], k[0][2]}, {k[1][0], k[1][1], k[1][2]}}, has_window, C::BM, C::BN,
                     C::BK, C::WM, C::WN, C::KG, C::THREADS, C::OCC, C::STAGE_BYTES, C::POLICY, C::BUDGET, cost};
}

inline void fill_static(const VariantDesc& v, int idx, gemm_w4a4_plan_t* pl) {
  memset(pl, 0, sizeof(*pl));
  pl->variant = idx;
  pl->block_m = v.block_m;
  pl->block_n = v.block_n;
  pl->block_k = v.block_k;
  pl->stages = v.budget.depth;
  pl->waves_m = v.waves_m;
  pl->waves_n = v.waves_n;
  pl->k_groups = v.k_groups;
  pl->threads = v.threads;
  pl->lds_bytes = v.budget.lds_bytes;
  pl->lds_stage_bytes = v.stage_bytes;
  pl->lds_limit = kLdsLimit;
  pl->occupancy = v.occ;
  pl->policy = v.policy;
  pl->lora_place = v.budget.place;
  pl->lds_ring_bytes = v.budget.ring_bytes;
  pl->lds_side_bytes = v.budget.side_bytes;
  // registers a lane may hold: 512 (VGPR + AGPR) per SIMD lane, shared by the
  // waves resident on that SIMD
  const int waves_per_simd = std::max(1, (v.waves_m * v.waves_n * v.k_groups * v.occ + 3) / 4);
  pl->regs_limit = 512 / waves_per_simd;
  pl->flavour = -1;
  pl->vgprs = pl->agprs = pl->sgprs = -1;
}

// Registers of the kernel a launch of flavour `flavour` would run (bf16 output).
inline void fill_registers(const VariantDesc& v, int flavour, gemm_w4a4_plan_t* pl) {
  pl->flavour = flavour;
  if (const KernelResources* r = find_resources(v.kernel[0][flavour])) {
    pl->vgprs = r->vgpr;
    pl->agprs = r->agpr;
    pl->sgprs = r->sgpr;
  }
}

// The solver's choice among compiled instances: for each, the rounds the chip
// needs (tiles / (CUs x workgroups resident per CU)) times the time of one
// round (workgroups on the busiest CU x tile elements x the instance's cost
// per element); the smallest estimate wins, ties to the earlier instance.
inline int choose_variant(const VariantDesc* vs, int n, int M, int N) {
  int best = 0;
  double best_cost = 0.0;
  for (int i = 0; i < n; ++i) {
    const VariantDesc& x = vs[i];
    const long tiles = long((M + x.block_m - 1) / x.block_m) * long((N + x.block_n - 1) / x.block_n);
    const long slots = long(kNumCUs) * x.occ;
    const long rounds = (tiles + slots - 1) / slots;
    const long per_cu = std::min<long>(x.occ, (tiles + kNumCUs - 1) / kNumCUs);
    const double cost = double(rounds) * double(per_cu) * x.block_m * x.block_n * x.cost;
    if (i == 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  return best;
}

// Problem-size part of a plan for instance `v` (index `idx`).
inline int plan_for(const VariantDesc& v, int idx, int M, int N, int K, int R, gemm_w4a4_plan_t* pl) {
  fill_static(v, idx, pl);
  pl->tiles_m = (M + v.block_m - 1) / v.block_m;
  pl->tiles_n = (N + v.block_n - 1) / v.block_n;
  const long grid = long(pl->tiles_m) * pl->tiles_n;
  if (grid > 0x7fffffffL) return GEMM_W4A4_EINVAL;
  pl->grid = int(grid);
  pl->k_stages = (K + v.block_k - 1) / v.block_k;
  pl->lora_steps = (R + 15) / 16;
  return GEMM_W4A4_OK;
}

// Arguments of one operator call, as the entry points receive them.
struct CallArgs {
  const uint8_t *act, *ascales, *wgt, *wscales;
  const float *wcscale, *bias;
  const uint16_t *lora_act_in, *lora_up;
  uint16_t* out;
  int M, N, K, R;
  void* stream;
};

// Pointer, alignment and overlap checks shared by both formats (sizes are
// checked by the caller); `block` is the k-width of one scale.
inline int check_call(const CallArgs& a, int block) {
  if (!a.act || !a.ascales || !a.wgt || !a.wscales || !a.wcscale || !a.bias || !a.out) return GEMM_W4A4_EINVAL;
  if (a.R > 0 && (!a.lora_act_in || !a.lora_up)) return GEMM_W4A4_EINVAL;
  if ((uintptr_t(a.act) | uintptr_t(a.wgt)) & 15u) return GEMM_W4A4_EALIGN;
  if ((uintptr_t(a.wcscale) | uintptr_t(a.bias)) & 3u) return GEMM_W4A4_EALIGN;
  if ((uintptr_t(a.out) | (a.R > 0 ? (uintptr_t(a.lora_act_in) | uintptr_t(a.lora_up)) : 0u)) & 1u)
    return GEMM_W4A4_EALIGN;
  const size_t Ms = size_t(a.M), Ns = size_t(a.N), Ks = size_t(a.K), Rs = size_t(a.R);
  const size_t out_bytes = Ms * Ns * 2;
  const struct { const void* p; size_t n; } ins[] = {
      {a.act, Ms * Ks / 2},        {a.ascales, Ks / block * Ms}, {a.wgt, Ns * Ks / 2},
      {a.wscales, Ks / block * Ns}, {a.wcscale, Ns * 4},          {a.bias, Ns * 4},
      {a.lora_act_in, Ms * Rs * 2}, {a.lora_up, Rs * Ns * 2}};
  for (const auto& in : ins)
    if (overlaps(a.out, out_bytes, in.p, in.n)) return GEMM_W4A4_EOVERLAP;
  return GEMM_W4A4_OK;
}

inline int launch_kernel(const void* kernel, const gemm_w4a4_plan_t& pl, const CallArgs& a) {
  Params prm;
  prm.act = a.act;
  prm.ascales = a.ascales;
  prm.wgt = a.wgt;
  prm.wscales = a.wscales;
  prm.wcscale = a.wcscale;
  prm.bias = a.bias;
  prm.lora_act_in = a.lora_act_in;
  prm.lora_up = a.lora_up;
  prm.out = a.out;
  prm.M = a.M;
  prm.N = a.N;
  prm.K = a.K;
  prm.R = a.R;
  prm.tiles_m = pl.tiles_m;
  prm.tiles_n = pl.tiles_n;
  void* args[] = {&prm};
  const hipError_t e = hipLaunchKernel(kernel, dim3(pl.grid), dim3(pl.threads), args, 0,
                                       static_cast<hipStream_t>(a.stream));
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}

}  // namespace w4a4
