// gemm_w4a4.hip — fused NVFP4 W4A4 GEMM + per-column affine + rank-R LoRA for gfx950.
//
// y[m,n] = wcscale[n] * sum_k A[m,k] W[n,k] + bias[n] + sum_r la[m,r] lu[r,n]
// (operator and formats: the SVDQuant W4A4 on Blackwell page, sections 2, 3.1
// and 6.6; E2M1 bit layout: the DeepGEMM FP4 indexer page, "Step 0").
//
// Design (one workgroup per BM x BN output tile, WM x WN waves):
//  * Loader: each K stage (128 values of k = 64 packed bytes per row) of act
//    and wgt is read from HBM with coalesced 16-byte loads into registers one
//    stage ahead, then written into an LDS ring whose 16-byte chunks are XOR
//    swizzled by row so that the consumer's 128-bit LDS reads do not conflict.
//  * Decode: NVFP4 is exact in fp16. Every E2M1 value times every E4M3 scale
//    has at most 6 significant bits and lies in [2^-10, 2688], so each operand
//    value is built exactly as fp16: v_cvt_scalef32_pk_f16_fp4 (scale 1.0)
//    turns two nibbles into two fp16 values and one packed fp16 multiply by
//    the (s, s) scale pair applies the block scale. The E4M3 -> fp16 scale
//    conversion is a 256-entry table in LDS, built once per workgroup with
//    integer arithmetic.
//  * K-loop: v_mfma_f32_32x32x16_f16, whose 16-deep k-step is exactly one
//    NVFP4 scale block. Each lane feeds 8 values of k that share one scale.
//    The k <-> MFMA-slot assignment is free as long as both operands use the
//    same one (the sum over k does not depend on its order), so a lane takes
//    the 8 nibbles of one packed dword.
//  * Epilogue: acc *= wcscale[n]; then the LoRA-up product runs as further
//    k-steps of the same-shape MFMA (v_mfma_f32_32x32x16_bf16, identical
//    accumulator layout) into the same accumulators; then + bias[n], bf16
//    round-to-nearest-even, masked store of rows < M and columns < N.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "gemm_w4a4.h"
#include "w4a4_layout.hpp"

namespace w4a4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
  int tiles_n;
};

// 16-byte chunk c of a row is stored at chunk position c ^ swz(row). Rows are
// 64 bytes apart, so without it rows r and r+2 (32 banks) or r and r+4
// (64 banks) would share banks under a 128-bit read; this XOR spreads any 8
// (or 16) consecutive rows of one chunk over distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// E4M3FN byte -> fp16 bit pattern. Exact: every E4M3 value is zero, NaN or an
// fp16 normal number (the smallest E4M3 subnormal, 2^-9, is above fp16's 2^-14).
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  uint32_t h;
  if (e == 15u && m == 7u) {
    h = 0x7E00u;                                     // NaN
  } else if (e == 0u) {
    if (m == 0u) {
      h = 0u;
    } else {                                         // m * 2^-9 = 2^(p-9) * (m / 2^p)
      const uint32_t p = 31u - __builtin_clz(m);
      h = ((p + 6u) << 10) | ((m - (1u << p)) << (10u - p));
    }
  } else {                                           // 2^(e-7) * (1 + m/8)
    h = ((e + 8u) << 10) | (m << 7);
  }
  return (s << 15) | h;
}

// Eight E2M1 nibbles of one dword, times the block scale pair (s, s), as fp16.
// Which nibble lands in which of the eight slots is irrelevant (see the file
// comment); both operands go through this same function.
__device__ __forceinline__ f16x8 decode8(uint32_t w, uint32_t scale_pair) {
  const f16x2 s = __builtin_bit_cast(f16x2, scale_pair);
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// One 16-byte chunk of a packed row, zero past the row end. Rows are a
// multiple of 8 bytes (K % 16 == 0); VEC16 says they are a multiple of 16.
template <bool VEC16>
__device__ __forceinline__ u32x4 load_chunk(const uint8_t* rowp, int kbyte, int rowbytes) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (kbyte + 16 <= rowbytes) {
    if constexpr (VEC16) {
      v = *reinterpret_cast<const u32x4*>(rowp + kbyte);
    } else {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(rowp + kbyte);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(rowp + kbyte + 8);
      v = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  } else if (kbyte + 8 <= rowbytes) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(rowp + kbyte);
    v.x = lo.x;
    v.y = lo.y;
  }
  return v;
}

__device__ __forceinline__ uint32_t bf16_pair(uint16_t lo, uint16_t hi) {
  return uint32_t(lo) | (uint32_t(hi) << 16);
}

template <class C, bool VEC16>
__global__ __launch_bounds__(C::THREADS) void gemm_w4a4_kernel(const Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem + C::LUT_OFF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;                 // which half of the wave (k group)
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const int tile = blockIdx.x;
  const int tm = tile / p.tiles_n, tn = tile % p.tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int M = p.M, N = p.N, K = p.K, R = p.R;
  const int rowbytes = K >> 1;
  const int KB = K >> 4;                   // scale blocks along k
  const int nst = (K + C::BK - 1) / C::BK;

  if (tid < 256) {
    const uint32_t h = e4m3_to_f16_bits(uint32_t(tid));
    lut[tid] = h | (h << 16);
  }

  // Byte offsets (32-bit: every tensor is below 2^31 bytes) of the rows of
  // act and wgt this thread copies into LDS. Rows past M or N are clamped
  // into range: they are loaded but their outputs are never stored.
  uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
#pragma unroll
  for (int u = 0; u < C::A_LOADS; ++u) {
    const int q = tid + u * C::THREADS;
    const int row = q >> 2;
    const int c = (q & 3) ^ swz(row);
    a_off[u] = uint32_t(min(m0 + row, M - 1)) * uint32_t(rowbytes) + uint32_t(c * 16);
  }
#pragma unroll
  for (int u = 0; u < C::B_LOADS; ++u) {
    const int q = tid + u * C::THREADS;
    const int row = q >> 2;
    const int c = (q & 3) ^ swz(row);
    b_off[u] = uint32_t(min(n0 + row, N - 1)) * uint32_t(rowbytes) + uint32_t(c * 16);
  }

  // Rows / columns of this lane's MFMA tiles (for scales and the epilogue).
  int arow[C::MI], bcol[C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) arow[i] = min(m0 + wm * C::TM + 32 * i + l32, M - 1);
#pragma unroll
  for (int j = 0; j < C::NI; ++j) bcol[j] = min(n0 + wn * C::TN + 32 * j + l32, N - 1);
  // lane half g reads scale blocks st*8 + 4g + q (q = 0..3) of stage st
  const uint32_t sa_lane = uint32_t(g * C::QS) * uint32_t(M);
  const uint32_t sb_lane = uint32_t(g * C::QS) * uint32_t(N);

  u32x4 pa[C::A_LOADS], pb[C::B_LOADS];
  uint32_t sa_b[C::MI][C::QS], sb_b[C::NI][C::QS];

  // FULL: the whole stage lies inside K (every stage but a partial last one),
  // so no chunk needs a bounds check.
  auto load_stage = [&]<bool FULL>(int st) {
    const uint32_t kbyte0 = uint32_t(st * C::ROW_BYTES);
    if constexpr (FULL) {
#pragma unroll
      for (int u = 0; u < C::A_LOADS; ++u)
        pa[u] = *reinterpret_cast<const u32x4*>(p.act + (a_off[u] + kbyte0));
#pragma unroll
      for (int u = 0; u < C::B_LOADS; ++u)
        pb[u] = *reinterpret_cast<const u32x4*>(p.wgt + (b_off[u] + kbyte0));
    } else {
      // chunk position inside its row = offset modulo the row length
#pragma unroll
      for (int u = 0; u < C::A_LOADS; ++u) {
        const uint32_t o = a_off[u] + kbyte0;
        const uint32_t in_row = ((tid + u * C::THREADS) & 3 ^ swz((tid + u * C::THREADS) >> 2)) * 16 + kbyte0;
        pa[u] = load_chunk<VEC16>(p.act + (o - in_row), int(in_row), rowbytes);
      }
#pragma unroll
      for (int u = 0; u < C::B_LOADS; ++u) {
        const uint32_t o = b_off[u] + kbyte0;
        const uint32_t in_row = ((tid + u * C::THREADS) & 3 ^ swz((tid + u * C::THREADS) >> 2)) * 16 + kbyte0;
        pb[u] = load_chunk<VEC16>(p.wgt + (o - in_row), int(in_row), rowbytes);
      }
    }
#pragma unroll
    for (int q = 0; q < C::QS; ++q) {
      const int kb = st * C::KSTEPS + g * C::QS + q;
      const bool ok = FULL || kb < KB;
      const uint32_t oa = ok ? uint32_t(st * C::KSTEPS + q) * uint32_t(M) + sa_lane : 0u;
      const uint32_t ob = ok ? uint32_t(st * C::KSTEPS + q) * uint32_t(N) + sb_lane : 0u;
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const uint32_t v = p.ascales[oa + uint32_t(arow[i])];
        sa_b[i][q] = ok ? v : 0u;
      }
#pragma unroll
      for (int j = 0; j < C::NI; ++j) {
        const uint32_t v = p.wscales[ob + uint32_t(bcol[j])];
        sb_b[j][q] = ok ? v : 0u;
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* base = smem + C::RING_OFF + buf * C::STAGE_BYTES;
#pragma unroll
    for (int u = 0; u < C::A_LOADS; ++u)
      *reinterpret_cast<u32x4*>(base + (tid + u * C::THREADS) * 16) = pa[u];
#pragma unroll
    for (int u = 0; u < C::B_LOADS; ++u)
      *reinterpret_cast<u32x4*>(base + C::A_BYTES + (tid + u * C::THREADS) * 16) = pb[u];
  };
  const int full_stages = rowbytes / C::ROW_BYTES;   // stages entirely inside K
  auto load_any = [&](int st) {
    if (st < full_stages) load_stage.template operator()<true>(st);
    else load_stage.template operator()<false>(st);
  };

  f32x16 acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_any(0);
  store_stage(0);
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st % C::STAGES;
    // block scales of this stage -> (s, s) fp16 pairs
    uint32_t sa[C::MI][C::QS], sb[C::NI][C::QS];
#pragma unroll
    for (int q = 0; q < C::QS; ++q) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i) sa[i][q] = lut[sa_b[i][q]];
#pragma unroll
      for (int j = 0; j < C::NI; ++j) sb[j][q] = lut[sb_b[j][q]];
    }
    if (st + 1 < nst) load_any(st + 1);

    // this lane's packed bytes: row l32 of each tile, chunks 2g and 2g+1
    const uint8_t* base = smem + C::RING_OFF + buf * C::STAGE_BYTES;
    uint32_t a[C::MI][8], b[C::NI][8];
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int row = wm * C::TM + 32 * i + l32;
      const uint8_t* rp = base + row * C::ROW_BYTES;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(rp + (((2 * g) ^ swz(row)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(rp + (((2 * g + 1) ^ swz(row)) << 4));
      a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
      a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      const int row = wn * C::TN + 32 * j + l32;
      const uint8_t* rp = base + C::A_BYTES + row * C::ROW_BYTES;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(rp + (((2 * g) ^ swz(row)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(rp + (((2 * g + 1) ^ swz(row)) << 4));
      b[j][0] = lo.x; b[j][1] = lo.y; b[j][2] = lo.z; b[j][3] = lo.w;
      b[j][4] = hi.x; b[j][5] = hi.y; b[j][6] = hi.z; b[j][7] = hi.w;
    }

    // k-step s uses dword s of the lane's 32 bytes: k = 64*g + 8*s + (0..7),
    // all inside scale block 4*g + s/2 of this stage.
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      f16x8 av[C::MI], bv[C::NI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i) av[i] = decode8(a[i][s], sa[i][s >> 1]);
#pragma unroll
      for (int j = 0; j < C::NI; ++j) bv[j] = decode8(b[j][s], sb[j][s >> 1]);
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }

    if (st + 1 < nst) store_stage((st + 1) % C::STAGES);
    __syncthreads();
  }

  // ---------------- epilogue: *wcscale, + LoRA (same accumulators), + bias, bf16 store
  float wc[C::NI], bs[C::NI];
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    wc[j] = p.wcscale[bcol[j]];
    bs[j] = p.bias[bcol[j]];
  }
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= wc[j];

  // LoRA-up: ceil(R/16) further k-steps into the same accumulators. Lane
  // (row l32, half g) feeds ranks rb .. rb+7 with rb = r0 + 8g; ranks past R
  // read a clamped address and are replaced by zero (no branches).
  const bool la_vec = (R & 7) == 0 && (reinterpret_cast<uintptr_t>(p.lora_act_in) & 15u) == 0;
  for (int r0 = 0; r0 < R; r0 += 16) {
    bf16x8 la[C::MI], lu[C::NI];
    const int rb = r0 + 8 * g;
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const uint16_t* src = p.lora_act_in + uint32_t(arow[i]) * uint32_t(R);
      if (la_vec) {
        // R % 8 == 0 and rb % 8 == 0: the eight ranks are all in range or all out
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + min(rb, R - 8));
        la[i] = __builtin_bit_cast(bf16x8, rb < R ? v : u32x4{0u, 0u, 0u, 0u});
      } else {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = rb + 2 * t;
          const uint16_t x0 = src[min(r, R - 1)];
          const uint16_t x1 = src[min(r + 1, R - 1)];
          w[t] = bf16_pair(r < R ? x0 : uint16_t(0), r + 1 < R ? x1 : uint16_t(0));
        }
        la[i] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      }
    }
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      const uint16_t* src = p.lora_up + bcol[j];
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = rb + 2 * t;
        const uint16_t x0 = src[uint32_t(min(r, R - 1)) * uint32_t(N)];
        const uint16_t x1 = src[uint32_t(min(r + 1, R - 1)) * uint32_t(N)];
        w[t] = bf16_pair(r < R ? x0 : uint16_t(0), r + 1 < R ? x1 : uint16_t(0));
      }
      lu[j] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lu[j], acc[i][j], 0, 0, 0);
  }

  // accumulator element r of a 32x32 tile: row 8*(r/4) + 4*g + r%4, column l32
  __bf16* out = reinterpret_cast<__bf16*>(p.out);
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      const int col = n0 + wn * C::TN + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::TM + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < M && col < N) out[size_t(row) * N + col] = __bf16(acc[i][j][r] + bs[j]);
      }
    }
  }
}

// ------------------------------------------------------------------ host side

struct Variant {
  void (*kernel[2])(const Params);   // [rows 16-byte multiple]
  int block_m, block_n, block_k, stages, waves_m, waves_n, threads, lds_bytes, stage_bytes, occ;
};

template <class C>
constexpr Variant make_variant() {
  return Variant{{gemm_w4a4_kernel<C, false>, gemm_w4a4_kernel<C, true>},
                 C::BM, C::BN, C::BK, C::STAGES, C::WM, C::WN, C::THREADS,
                 C::LDS_BYTES, C::STAGE_BYTES, C::OCC};
}

static const Variant kVariants[] = {make_variant<Cfg256x192>(), make_variant<Cfg128x128>()};
static constexpr int kNumVariants = int(sizeof(kVariants) / sizeof(kVariants[0]));

static void fill_static(const Variant& v, int idx, gemm_w4a4_plan_t* pl) {
  memset(pl, 0, sizeof(*pl));
  pl->variant = idx;
  pl->block_m = v.block_m;
  pl->block_n = v.block_n;
  pl->block_k = v.block_k;
  pl->stages = v.stages;
  pl->waves_m = v.waves_m;
  pl->waves_n = v.waves_n;
  pl->threads = v.threads;
  pl->lds_bytes = v.lds_bytes;
  pl->lds_stage_bytes = v.stage_bytes;
  pl->lds_limit = kLdsLimit;
}

// Size rules. Besides the operator's own (K a multiple of the 16-wide scale
// block), every tensor must stay below 2^31 bytes: the kernels address them
// with 32-bit offsets from a uniform base.
static bool sizes_ok(int M, int N, int K, int R) {
  if (!(M >= 1 && N >= 1 && K >= 16 && K % 16 == 0 && R >= 0 && R <= GEMM_W4A4_MAX_R))
    return false;
  const int64_t lim = int64_t(1) << 31;
  const int64_t m = M, n = N, k = K, r = R;
  return m * k / 2 < lim && n * k / 2 < lim && m * n * 2 < lim && m * r * 2 < lim &&
         r * n * 2 < lim;
}

// Budget solver: for each compiled instance, the number of rounds the chip
// needs (tiles / (CUs * workgroups resident per CU)) times the time of one
// round (the resident workgroups share the CU, so occ tiles of work); picks
// the instance with the smallest estimate. Ties go to the earlier, larger
// tile, whose decode cost per flop is lower.
static int choose_variant(int M, int N) {
  int best = 0;
  double best_cost = 0.0;
  for (int v = 0; v < kNumVariants; ++v) {
    const Variant& x = kVariants[v];
    const long tiles = long((M + x.block_m - 1) / x.block_m) * long((N + x.block_n - 1) / x.block_n);
    const long slots = long(kNumCUs) * x.occ;
    const long rounds = (tiles + slots - 1) / slots;
    // relative throughput of one resident workgroup: decode VALU per MFMA grows
    // as (TM + TN) / (TM * TN) for a wave tile TM x TN
    const double tm = double(x.block_m / x.waves_m), tn = double(x.block_n / x.waves_n);
    const double decode = 8.0 * 4.0 * (tm + tn) / (tm * tn);   // VALU cycles per MFMA cycle
    const double per_round = double(x.occ) * x.block_m * x.block_n * (1.0 + 0.5 * decode);
    const double cost = double(rounds) * per_round;
    if (v == 0 || cost < best_cost) {
      best = v;
      best_cost = cost;
    }
  }
  return best;
}

static int plan_impl(int M, int N, int K, int R, gemm_w4a4_plan_t* pl) {
  const int v = choose_variant(M, N);
  const Variant& x = kVariants[v];
  fill_static(x, v, pl);
  pl->tiles_m = (M + x.block_m - 1) / x.block_m;
  pl->tiles_n = (N + x.block_n - 1) / x.block_n;
  const long grid = long(pl->tiles_m) * pl->tiles_n;
  if (grid > 0x7fffffffL) return GEMM_W4A4_EINVAL;
  pl->grid = int(grid);
  pl->k_stages = (K + x.block_k - 1) / x.block_k;
  pl->lora_steps = (R + 15) / 16;
  return GEMM_W4A4_OK;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = uintptr_t(a), y = uintptr_t(b);
  return x < y + nb && y < x + na;
}

static std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, 2 other

static int check_device() {
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

using namespace w4a4;

extern "C" int gemm_w4a4_plan(int M, int N, int K, int R, gemm_w4a4_plan_t* plan) {
  if (!plan || !sizes_ok(M, N, K, R)) return GEMM_W4A4_EINVAL;
  return plan_impl(M, N, K, R, plan);
}

extern "C" int gemm_w4a4_num_variants(void) { return kNumVariants; }

extern "C" int gemm_w4a4_variant_info(int variant, gemm_w4a4_plan_t* plan) {
  if (!plan || variant < 0 || variant >= kNumVariants) return GEMM_W4A4_EINVAL;
  fill_static(kVariants[variant], variant, plan);
  return GEMM_W4A4_OK;
}

extern "C" const char* gemm_w4a4_strerror(int code) {
  switch (code) {
    case GEMM_W4A4_OK: return "success";
    case GEMM_W4A4_EINVAL: return "invalid argument (size or NULL pointer)";
    case GEMM_W4A4_EALIGN: return "misaligned pointer";
    case GEMM_W4A4_ELAUNCH: return "HIP kernel launch failed";
    case GEMM_W4A4_EOVERLAP: return "output overlaps an input";
    case GEMM_W4A4_EDEVICE: return "current device is not gfx950";
    default: return "unknown error";
  }
}

extern "C" int gemm_w4a4(const uint8_t* act, const uint8_t* ascales, const uint8_t* wgt,
                         const uint8_t* wscales, const float* wcscale, const float* bias,
                         const uint16_t* lora_act_in, const uint16_t* lora_up, uint16_t* out,
                         int M, int N, int K, int R, void* stream) {
  if (!sizes_ok(M, N, K, R)) return GEMM_W4A4_EINVAL;
  if (!act || !ascales || !wgt || !wscales || !wcscale || !bias || !out) return GEMM_W4A4_EINVAL;
  if (R > 0 && (!lora_act_in || !lora_up)) return GEMM_W4A4_EINVAL;
  if ((uintptr_t(act) | uintptr_t(wgt)) & 15u) return GEMM_W4A4_EALIGN;
  if ((uintptr_t(wcscale) | uintptr_t(bias)) & 3u) return GEMM_W4A4_EALIGN;
  if ((uintptr_t(out) | (R > 0 ? (uintptr_t(lora_act_in) | uintptr_t(lora_up)) : 0u)) & 1u)
    return GEMM_W4A4_EALIGN;

  const size_t Ms = size_t(M), Ns = size_t(N), Ks = size_t(K), Rs = size_t(R);
  const size_t out_bytes = Ms * Ns * 2;
  const struct { const void* p; size_t n; } ins[] = {
      {act, Ms * Ks / 2},     {ascales, Ks / 16 * Ms}, {wgt, Ns * Ks / 2},
      {wscales, Ks / 16 * Ns}, {wcscale, Ns * 4},      {bias, Ns * 4},
      {lora_act_in, Ms * Rs * 2}, {lora_up, Rs * Ns * 2}};
  for (const auto& in : ins)
    if (overlaps(out, out_bytes, in.p, in.n)) return GEMM_W4A4_EOVERLAP;

  gemm_w4a4_plan_t pl;
  if (plan_impl(M, N, K, R, &pl) != GEMM_W4A4_OK) return GEMM_W4A4_EINVAL;
  const int dev_rc = check_device();
  if (dev_rc != GEMM_W4A4_OK) return dev_rc;

  Params prm;
  prm.act = act;
  prm.ascales = ascales;
  prm.wgt = wgt;
  prm.wscales = wscales;
  prm.wcscale = wcscale;
  prm.bias = bias;
  prm.lora_act_in = lora_act_in;
  prm.lora_up = lora_up;
  prm.out = out;
  prm.M = M;
  prm.N = N;
  prm.K = K;
  prm.R = R;
  prm.tiles_n = pl.tiles_n;

  const Variant& v = kVariants[pl.variant];
  const bool vec16 = ((K / 2) % 16) == 0;
  void* args[] = {&prm};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(v.kernel[vec16 ? 1 : 0]),
                                       dim3(pl.grid), dim3(v.threads), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}
