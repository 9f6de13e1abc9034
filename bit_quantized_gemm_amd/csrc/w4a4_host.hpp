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
  pl->tail_variant = -1;
  pl->tail_splits = 1;
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

// The solver's estimate for instance x over `rows` rows: the rounds the chip
// needs (tiles / (CUs x workgroups resident per CU)) times the time of one
// round (workgroups on the busiest CU x tile elements x the instance's cost
// per element).
inline double estimate(const VariantDesc& x, int rows, int N) {
  const long tiles = long((rows + x.block_m - 1) / x.block_m) * long((N + x.block_n - 1) / x.block_n);
  const long slots = long(kNumCUs) * x.occ;
  const long rounds = (tiles + slots - 1) / slots;
  const long per_cu = std::min<long>(x.occ, (tiles + kNumCUs - 1) / kNumCUs);
  return double(rounds) * double(per_cu) * x.block_m * x.block_n * x.cost;
}

// The solver's choice among compiled instances: the smallest estimate of one
// instance over all M rows (ties to the earlier instance), or of a main
// instance over its first M1 rows followed by a second launch of a tail
// instance over the last M - M1 rows. M1 is a whole number of the main
// instance's tile rows: those of its whole rounds (k times the tile rows one
// round holds), or all of its whole tile rows when M is not a multiple of
// its BM. The tail instance's BM divides the main one's, so its first tile
// row M1 / BM_tail is whole. At M = 17 x 256 rows this runs 16 tile rows of
// 256 x 192 in one round and the 17th on 64-row tiles, instead of a second
// round for 16 tiles or a smaller tile everywhere.
//
// The estimate has no K: it counts rounds of k-loops. Every launch past the
// first adds what a launch costs besides its k-loop (ring fill, epilogue, the
// store of its tiles), about `launch_stages` k-stages of a full round of
// instance 0, so each candidate pays that share of a round of K/128 stages
// per extra launch.
//
// K slices: when `part` (an instance compiled with K-sliced workgroups, -1
// for none) is the tail instance, the tail may instead run its K in S slices
// over S times the workgroups (one round), writing float32 sums that a
// reduction launch adds. Its rows take 1/S of the tail's estimate and two
// extra launches. The sums live in the main launch's rows of the output,
// which that launch, enqueued after the reduction, overwrites, so a slice
// count needs S x tail rows x 4 bytes <= M1 x 2 bytes; 2 <= S <= 8, and every
// slice keeps at least two stages.
struct Choice {
  int main, tail;   // instances; tail -1: one launch over all M rows
  int main_rows;    // rows of the main launch (M when there is no tail)
  int splits;       // K slices of the tail (1: the tail runs whole)
};
inline Choice choose_plan(const VariantDesc* vs, int n, int M, int N, int K, double launch_stages, int part) {
  const double round0 = double(vs[0].occ) * vs[0].block_m * vs[0].block_n * vs[0].cost;
  const int nst = (K + vs[0].block_k - 1) / vs[0].block_k;
  const double launch = launch_stages / double(nst) * round0;   // one extra launch
  Choice best{0, -1, M, 1};
  double best_cost = estimate(vs[0], M, N);
  auto take = [&](const Choice& c, double cost) {
    if (cost < best_cost) {
      best = c;
      best_cost = cost;
    }
  };
  for (int i = 1; i < n; ++i) take(Choice{i, -1, M, 1}, estimate(vs[i], M, N));
  auto consider = [&](int i, int m1) {
    if (m1 <= 0 || m1 >= M) return;
    const double main = estimate(vs[i], m1, N);
    for (int j = 0; j < n; ++j) {
      if (vs[i].block_m % vs[j].block_m != 0) continue;
      const int rows = M - m1;
      const double tail = estimate(vs[j], rows, N);
      take(Choice{i, j, m1, 1}, main + tail + launch);
      if (j != part) continue;
      const long tiles = long((rows + vs[j].block_m - 1) / vs[j].block_m) * ((N + vs[j].block_n - 1) / vs[j].block_n);
      const long fit = std::min<long>({8, long(kNumCUs) * vs[j].occ / tiles, long(nst) / 2, long(m1) / (2L * rows)});
      if (fit >= 2) take(Choice{i, j, m1, int(fit)}, main + tail / double(fit) + 2.0 * launch);
    }
  };
  for (int i = 0; i < n; ++i) {
    const VariantDesc& x = vs[i];
    consider(i, M / x.block_m * x.block_m);
    const long round_rows = long(kNumCUs) * x.occ / ((N + x.block_n - 1) / x.block_n);   // tile rows a round holds
    for (long k = 1; round_rows > 0 && k <= 64 && k * round_rows * x.block_m < M; ++k)
      consider(i, int(k * round_rows * x.block_m));
  }
  return best;
}

// Problem-size part of a plan for instance `v` (index `idx`) over the first
// `rows` of the M rows (all of them, or a split's main launch).
inline int plan_for(const VariantDesc& v, int idx, int rows, int N, int K, int R, gemm_w4a4_plan_t* pl) {
  fill_static(v, idx, pl);
  pl->tiles_m = (rows + v.block_m - 1) / v.block_m;
  pl->tiles_n = (N + v.block_n - 1) / v.block_n;
  const long grid = long(pl->tiles_m) * pl->tiles_n;
  if (grid > 0x7fffffffL) return GEMM_W4A4_EINVAL;
  pl->grid = int(grid);
  pl->k_stages = (K + v.block_k - 1) / v.block_k;
  pl->lora_steps = (R + 15) / 16;
  pl->tail_variant = -1;
  pl->tail_rows = pl->tail_block_m = pl->tail_block_n = pl->tail_grid = 0;
  pl->tail_splits = 1;
  return GEMM_W4A4_OK;
}

// The plan of a solver choice `c` (its tail fields filled when it splits).
inline int plan_choice(const VariantDesc* vs, const Choice& c, int M, int N, int K, int R, gemm_w4a4_plan_t* pl) {
  const int rc = plan_for(vs[c.main], c.main, c.main_rows, N, K, R, pl);
  if (rc != GEMM_W4A4_OK || c.tail < 0) return rc;
  const VariantDesc& t = vs[c.tail];
  pl->tail_variant = c.tail;
  pl->tail_rows = M - c.main_rows;
  pl->tail_block_m = t.block_m;
  pl->tail_block_n = t.block_n;
  pl->tail_splits = c.splits;
  pl->tail_grid = (pl->tail_rows + t.block_m - 1) / t.block_m * ((N + t.block_n - 1) / t.block_n) * c.splits;
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

// One launch of `kernel` (instance v) over tile rows [tm0, tm0 + tiles_m) of
// its BM rows.
inline int launch_kernel(const void* kernel, const VariantDesc& v, int tiles_m, int tm0, const CallArgs& a,
                         int splits = 1, int part_rows = 0) {
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
  prm.tiles_m = tiles_m;
  prm.tiles_n = (a.N + v.block_n - 1) / v.block_n;
  prm.tm0 = tm0;
  // K slices: float32 sums over the rows before this launch's (see choose_plan)
  prm.part = splits > 1 ? reinterpret_cast<float*>(a.out) : nullptr;
  prm.part_row0 = tm0 * v.block_m;
  prm.part_rows = part_rows;
  void* args[] = {&prm};
  const hipError_t e = hipLaunchKernel(kernel, dim3(unsigned(long(tiles_m) * prm.tiles_n), unsigned(splits)),
                                       dim3(v.threads), args, 0, static_cast<hipStream_t>(a.stream));
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}

// A K-sliced tail: `part_kernel` (instance t, K-sliced workgroups) over the
// last `rows` rows in `splits` slices, its float32 sums in the output's first
// rows, then `reduce_kernel` (split_k_reduce of the output type) adding them
// into rows row0 .. row0 + rows - 1.
inline int launch_slices(const void* part_kernel, const void* reduce_kernel, const VariantDesc& t, int rows, int splits,
                         int row0, const CallArgs& a) {
  if (launch_kernel(part_kernel, t, (rows + t.block_m - 1) / t.block_m, row0 / t.block_m, a, splits, rows) !=
      GEMM_W4A4_OK)
    return GEMM_W4A4_ELAUNCH;
  const long groups = long(rows) * (a.N / 4);
  const float* part = reinterpret_cast<const float*>(a.out);
  uint16_t* out = a.out;
  int n = a.N, s = splits, r0 = row0, nr = rows;
  void* args[] = {&part, &out, &nr, &n, &s, &r0};
  return hipLaunchKernel(reduce_kernel, dim3(unsigned((groups + 255) / 256)), dim3(256), args, 0,
                         static_cast<hipStream_t>(a.stream)) == hipSuccess
             ? GEMM_W4A4_OK
             : GEMM_W4A4_ELAUNCH;
}

// The launches of a plan: the main instance, then the tail instance, if any,
// over the last rows (the same flavour rule; `kernel_of` maps an instance to
// the kernel of that flavour and output type). A K-sliced tail runs first:
// `sliced(rows, splits, row0)` enqueues its slices and their reduction, which
// use the main launch's rows of the output as scratch; the main launch then
// overwrites them. `sliced` returns GEMM_W4A4_EINVAL when the call's pointers
// do not allow slices; the tail then runs whole.
template <class KernelOf, class Sliced>
inline int launch_plan(const VariantDesc* vs, const gemm_w4a4_plan_t& pl, const CallArgs& a, KernelOf kernel_of,
                       Sliced sliced) {
  const VariantDesc& v = vs[pl.variant];
  const int main_rows = a.M - pl.tail_rows;
  bool tail_done = false;
  if (pl.tail_variant >= 0 && pl.tail_splits > 1) {
    const int rc = sliced(pl.tail_rows, pl.tail_splits, main_rows);
    if (rc == GEMM_W4A4_ELAUNCH) return rc;
    tail_done = rc == GEMM_W4A4_OK;
  }
  int rc = launch_kernel(kernel_of(v), v, pl.tiles_m, 0, a);
  if (rc != GEMM_W4A4_OK || pl.tail_variant < 0 || tail_done) return rc;
  const VariantDesc& t = vs[pl.tail_variant];
  return launch_kernel(kernel_of(t), t, (pl.tail_rows + t.block_m - 1) / t.block_m, main_rows / t.block_m, a);
}

}  // namespace w4a4
