// w4a4_producer.hip — the memory-bound half of SVDQuant W4A4 for gfx950: the
// bf16 activations x [M, K] quantised to the fused GEMM's NVFP4 operand (act
// [M, K/2], two E2M1 codes a byte, low nibble = even k; ascales [K/16, M], one
// FP8-E4M3 scale per 16 k) and the LoRA-down product lora_act_in [M, R] =
// x @ lora_down^T with lora_down [R, K]. The SVDQuant W4A4 on Blackwell page
// calls the GEMM the compute-bound half (section 1) and fixes these layouts
// (sections 2 and 3.1); the scale and rounding rule is this library's
// reading, stated in gemm_w4a4.h.
//
// Design (one workgroup of WAVES waves per 16 rows of x):
//  * x is read once. The workgroup's rows are cut into spans of 128 k; wave w
//    takes spans w, w+WAVES, ... and streams them through a private LDS ring
//    (DEPTH spans, 128 KiB / WAVES) by direct-to-LDS DMA, so the loop needs no
//    workgroup barrier. Each 256-byte row of a span is stored with its 16-byte
//    chunks XOR-swizzled by row, so that the reads below hit distinct banks.
//    More waves per workgroup (up to 16) keep every SIMD busy when M / 16 is
//    small. A span's lora_down operands are loaded at its start; their L2
//    latency hides behind the span's LDS read and quantisation.
//  * Lane (r, g) holds row r, k = 32g .. 32g+31 of the
//    span: two whole 16-value blocks, so a block's amax needs no cross-lane
//    step. Scale and codes are decided exactly (see quantize_block), codes are
//    packed by the FP4 conversion, act is written as 16 (or 2 x 8) bytes per
//    lane and the scale bytes are gathered through LDS into 16-byte rows of
//    ascales.
//  * The same registers are the A operand of v_mfma_f32_16x16x32_bf16: in
//    k-step i lane (r, g) supplies x[r][32g + 8i .. +7] and, as B operand,
//    lora_down[rank][32g + 8i .. +7] (any k order works if both sides agree).
//    The four waves' partial sums meet once through LDS at the end.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "gemm_w4a4.h"
#include "w4a4_common.hpp"
#include "w4a4_host.hpp"

namespace w4a4 {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// WAVES waves per 16-row workgroup, RTILES rank tiles of 16 (R <= 16 * RTILES).
template <int WAVES_, int RTILES_>
struct ProdCfg {
  static constexpr int WAVES = WAVES_, RTILES = RTILES_, RT = 1;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int ROWS = 16;
  static constexpr int SPAN_K = 128;
  static constexpr int TILE_BYTES = 16 * SPAN_K * 2;            // one 16-row tile of a span (4 KiB)
  static constexpr int SPAN_BYTES = TILE_BYTES;
  static constexpr int RING = 131072 / WAVES;                     // per wave
  static constexpr int DEPTH = RING / SPAN_BYTES;                 // spans in flight per wave
  static constexpr int SC_BYTES = 8 * ROWS;                       // staged scale bytes of a span
  static constexpr int SC_OFF = WAVES * RING;
  static constexpr int RED_BYTES = WAVES * RTILES * kWave * 16;   // end-of-loop partial sums
  static constexpr int LDS = SC_OFF + WAVES * SC_BYTES;
  static constexpr int D = SPAN_BYTES / (kWave * 16);             // 16-byte DMA rounds per span
  static constexpr int NL = 4 * RTILES;                           // lora_down loads per span
  // lora_down operands are loaded PL spans ahead into NSETS = PL + 1 register
  // sets (the span loop is unrolled NSETS times so that every set index is a
  // constant): as deep as the x ring for R <= 32; at the start of their own
  // span for the largest ranks, whose one set already takes half the
  // register file.
  static constexpr int PL = RTILES <= 2 ? (RTILES == 0 ? 0 : DEPTH - 1) : 0;
  static constexpr int NSETS = PL + 1;
  // Issue order: the prologue issues DMA(0 .. DEPTH-1) and L(0 .. PL-1); span
  // j issues the stores S(j-1) of the previous span's results, L(j + PL),
  // then the refill DMA(j + DEPTH) of its ring slot. Loads complete in issue
  // order (a store can only make a count of loads stricter), so waiting until
  // at most X vector-memory ops remain completes every load with at least X
  // younger loads:
  //   DMA(j): at least DEPTH-1 younger DMA groups and min(PL, DEPTH-1) L groups;
  //   L(j):   at least PL younger L groups and one DMA group.
  // (Counts above the counter's 63 are capped: a stricter wait.)
  static constexpr int VM_DMA = (DEPTH - 1) * D + (PL < DEPTH - 1 ? PL : DEPTH - 1) * NL < 63
                                    ? (DEPTH - 1) * D + (PL < DEPTH - 1 ? PL : DEPTH - 1) * NL : 63;
  static constexpr int VM_L = PL * NL + D < 63 ? PL * NL + D : 63;
  static_assert(DEPTH >= 2, "ring depth");
  static_assert(RED_BYTES <= WAVES * RING, "partial sums fit in the drained rings");
  static_assert(LDS <= kLdsLimit, "LDS budget");
};

struct ProdParams {
  const uint16_t* x;
  const uint16_t* lora_down;
  uint8_t* act;
  uint8_t* ascales;
  uint16_t* lora_act_in;
  int M, K, R;
};

// OCP E4M3FN byte of v, 0 <= v <= 448, rounded to nearest even (integer
// arithmetic on the float32 bits; below 2^-6 the subnormal grid m * 2^-9).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  // subnormal range: v * 2^9 + 2^23 rounds v * 2^9 to an integer, ties to even
  const uint32_t sub = __builtin_bit_cast(uint32_t, __builtin_fmaf(v, 512.0f, 8388608.0f)) - 0x4B000000u;
  // normal range: round the mantissa to 3 bits, ties to even; rebias 127 -> 7
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t nrm = ((r >> 20) - (120u << 3)) & 0xFFu;
  return v < 0.015625f ? sub : nrm;
}

// Value of an E4M3FN byte b in 0x00 .. 0x7E.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const float sub = float(b) * 0.001953125f;   // m * 2^-9
  const float nrm = __builtin_bit_cast(float, ((b + (120u << 3)) << 20));
  return b < 8u ? sub : nrm;
}

// One 16-value block (8 dwords of bf16 pairs) -> its scale byte and the 16
// codes packed as two dwords (low nibble first). Exact decisions:
//  * amax / 6: q = amax * fl(1/6) and one correction with the exact residual
//    fma(-q, 6, amax) return the exact quotient whenever it is a float32 (the
//    only case in which it can sit on an E4M3 midpoint: a tie) and otherwise
//    a value within an ulp of it, while every other quotient lies at least
//    2^-13 relative from every E4M3 midpoint; the integer rounding above is
//    exact.
//  * |x| / s: within 2^-22 relative of the exact quotient, which is either
//    exactly an E2M1 midpoint (a multiple of 0.25) or at least 2^-10 away from
//    every one; snapping to the 2^-12 grid (adding and subtracting 2048)
//    restores the exact midpoints and keeps every other quotient on its side,
//    so the conversion's nearest-even rounding decides like the exact one.
// A block holding a NaN or an infinity gets 0x7F and zero codes (computed
// branch-free: the arithmetic runs on whatever the block holds and is
// replaced at the end).
__device__ __forceinline__ void quantize_block(const uint32_t (&d)[8], uint32_t& sbyte, uint32_t& lo,
                                               uint32_t& hi) {
  // |x| bit patterns order like the magnitudes (NaN above infinity above
  // every finite value): a packed 16-bit max over the pairs, then the halves
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, d[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[i] & 0x7FFF7FFFu));
  const uint32_t amax_bits = max(uint32_t(m[0]), uint32_t(m[1]));
  const bool finite = amax_bits < 0x7F80u;
  const float amax = __builtin_bit_cast(float, (finite ? amax_bits : 0u) << 16);
  const float sixth = 1.0f / 6.0f;
  const float q0 = amax * sixth;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, amax), sixth, q0);
  const uint32_t sb = e4m3_rne(fminf(q, 448.0f));
  const float s = e4m3_value(sb);
  const float r = s > 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t xl = d[i] << 16, xh = d[i] & 0xFFFF0000u;
    // |x| * r snapped to the 2^-12 grid (never negative), then the sign of x
    const float ql = __builtin_fmaf(__builtin_fabsf(__builtin_bit_cast(float, xl)), r, 2048.0f) - 2048.0f;
    const float qh = __builtin_fmaf(__builtin_fabsf(__builtin_bit_cast(float, xh)), r, 2048.0f) - 2048.0f;
    const float sl = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, ql) | (xl & 0x80000000u));
    const float sh = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, qh) | (xh & 0x80000000u));
    // element 2i is k even (low nibble of byte i), 2i+1 odd; byte i of the 8
    switch (i & 3) {   // byte select must be an immediate; folds after unrolling
      case 0: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], sl, sh, 1.0f, 0); break;
      case 1: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], sl, sh, 1.0f, 1); break;
      case 2: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], sl, sh, 1.0f, 2); break;
      default: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], sl, sh, 1.0f, 3); break;
    }
  }
  sbyte = finite ? sb : 0x7Fu;
  lo = finite ? w[0] : 0u;
  hi = finite ? w[1] : 0u;
}

template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void producer_kernel(const ProdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, K = p.K, R = p.R;
  const int m0 = blockIdx.x * C::ROWS;
  const int nsp = (K + C::SPAN_K - 1) / C::SPAN_K;
  const int nmine = wave_u < nsp ? (nsp - 1 - wave_u) / C::WAVES + 1 : 0;   // spans of this wave
  const uint32_t row_bytes = uint32_t(K) * 2u;
  uint8_t* ring = smem + wave_u * C::RING;

  // DMA of this wave's j-th span into ring slot j % DEPTH. Round u:
  // lane l writes slot position (row 4u + l/16, chunk l%16) and reads data
  // chunk (l%16) ^ row of that row. Spans past the wave's last one re-read it
  // (never consumed); k past K and rows past M read clamped in-range bytes.
  auto dma_span = [&](int j) __attribute__((always_inline)) {
    const int jj = nmine > 0 ? min(j, nmine - 1) : 0;
    const int span = wave_u + C::WAVES * jj;
    uint8_t* slot = ring + (j % C::DEPTH) * C::SPAN_BYTES;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int lr = 4 * u + (lane >> 4);                         // row inside the tile
      const int row = min(m0 + lr, M - 1);
      const int chunk = (lane & 15) ^ lr;                         // 16-byte chunk = 8 k
      const int kk = span * C::SPAN_K + 8 * chunk;
      const uint32_t kb = kk < K ? uint32_t(kk) * 2u : 0u;
      dma<16>(reinterpret_cast<const uint8_t*>(p.x) + uint32_t(row) * row_bytes + kb, slot + u * 1024);
    }
  };

  f32x4_t acc[C::RTILES > 0 ? C::RTILES : 1];
#pragma unroll
  for (int jt = 0; jt < (C::RTILES > 0 ? C::RTILES : 1); ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LoRA-down operands of this wave's j-th span into register set `SET` (B:
  // lora_down[rank][k0 + 8i .. +7]); ranks past R re-read rank R-1 (their sums
  // are not stored), k past K re-reads the row's last 8 and is zeroed at use,
  // spans past the wave's last re-read that one (never used).
  //
  // Issued as explicit global_load_dwordx4, which the compiler does not track:
  // with stores in flight it would otherwise wait for every outstanding
  // vector-memory op (vmcnt(0)) before the first use, the ring's DMAs
  // included. The explicit waits below count loads only, and scheduling
  // fences keep every use after its wait.
  constexpr int LT = C::RTILES > 0 ? C::RTILES : 1;
  u32x4 lb[C::NSETS][LT][4];
  auto load_lora = [&](u32x4 (&dst)[LT][4], int j) __attribute__((always_inline)) {
    if constexpr (C::RTILES > 0) {
      const int jj = nmine > 0 ? min(j, nmine - 1) : 0;
      const int k0 = (wave_u + C::WAVES * jj) * C::SPAN_K + 32 * g;
#pragma unroll
      for (int jt = 0; jt < C::RTILES; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rank = min(16 * jt + r, R - 1);
          const int kk = min(k0 + 8 * i, K - 8);
          const uint16_t* src = p.lora_down + uint32_t(rank) * uint32_t(K) + uint32_t(kk);
          asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(dst[jt][i]) : "v"(src) : "memory");
        }
    }
  };

#pragma unroll
  for (int j = 0; j < C::DEPTH; ++j) dma_span(j);
  static_for<0, C::PL>([&]<int S>() __attribute__((always_inline)) { load_lora(lb[S], S); });

  const bool act16 = (K & 31) == 0 && (reinterpret_cast<uintptr_t>(p.act) & 15u) == 0;
  const bool sc16 = (M & 15) == 0 && (reinterpret_cast<uintptr_t>(p.ascales) & 15u) == 0;
  uint8_t* sc_stage = smem + C::SC_OFF + wave_u * C::SC_BYTES;

  // The results of a span are stored at the start of the next one, before its
  // lora_down loads and refill DMA, so that no store lies between a lora_down
  // load group and the ops its wait counts.
  uint32_t code[4] = {0u, 0u, 0u, 0u};   // the previous span's 32 codes of this lane
  u32x4 scv = {0u, 0u, 0u, 0u};          // lanes 0..7: one 16-byte row of its scales
  int prev_span = -1;
  auto store_span = [&]() __attribute__((always_inline)) {
    const int k0 = prev_span * C::SPAN_K + 32 * g;
    const bool ok0 = k0 < K, ok1 = k0 + 16 < K;
    const int row = m0 + r;
    if (row < M) {
      uint8_t* dst = p.act + uint32_t(row) * uint32_t(K / 2) + uint32_t(k0 / 2);
      if (act16 && ok1) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{code[0], code[1], code[2], code[3]};
      } else {
        if (ok0) *reinterpret_cast<u32x2*>(dst) = u32x2{code[0], code[1]};
        if (ok1) *reinterpret_cast<u32x2*>(dst + 8) = u32x2{code[2], code[3]};
      }
    }
    const int kb = prev_span * (C::SPAN_K / 16) + lane;
    if (lane < 8 && kb < K / 16) {
      uint8_t* dst = p.ascales + uint32_t(kb) * uint32_t(M) + uint32_t(m0);
      if (sc16 && m0 + 16 <= M) {
        *reinterpret_cast<u32x4*>(dst) = scv;
      } else {
        const uint32_t w4[4] = {scv.x, scv.y, scv.z, scv.w};
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (m0 + e < M) dst[e] = uint8_t(w4[e >> 2] >> (8 * (e & 3)));
      }
    }
  };

  // span j uses lora_down set j % NSETS; j0 is a multiple of NSETS
  auto one_span = [&]<int SET>(int j) __attribute__((always_inline)) {
    const int span = wave_u + C::WAVES * j;
    const int k0 = span * C::SPAN_K + 32 * g;                 // this lane's first k
    wait_vm_lgkm0<C::VM_DMA>();                               // DMA(j) has landed
    // scheduling fences keep the issue order the wait counts rely on
    __builtin_amdgcn_sched_barrier(0);
    if (prev_span >= 0) store_span();                         // S(j-1)
    __builtin_amdgcn_sched_barrier(0);
    load_lora(lb[(SET + C::PL) % C::NSETS], j + C::PL);      // L(j + PL)
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* slot = ring + (j % C::DEPTH) * C::SPAN_BYTES;
    uint32_t xd[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(slot + r * 256 + (((4 * g + i) ^ r) << 4));
      xd[4 * i] = v.x;
      xd[4 * i + 1] = v.y;
      xd[4 * i + 2] = v.z;
      xd[4 * i + 3] = v.w;
    }
    wait_vm_lgkm0<63>();                                      // the slot is read: refill it
    __builtin_amdgcn_sched_barrier(0);
    dma_span(j + C::DEPTH);
    __builtin_amdgcn_sched_barrier(0);
    // a span reaching past K (only the last, when K % 128 != 0): zero this
    // lane's blocks past K (they add nothing to the LoRA sums and are not stored)
    const bool tail = (span + 1) * C::SPAN_K > K;   // uniform
    if (tail) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (k0 + 16 * (i >> 3) >= K) xd[i] = 0u;
    }

    uint32_t sb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      uint32_t d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = xd[8 * b + i];
      quantize_block(d, sb[b], code[2 * b], code[2 * b + 1]);
    }

    if constexpr (C::RTILES > 0) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<C::VM_L>();                                     // L(j)
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");                          // nothing reads lb[SET] before this point
      if (tail) {
        // k past K: a zero operand (a NaN weight there must not reach valid sums)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jt = 0; jt < C::RTILES; ++jt)
            if (k0 + 8 * i >= K) lb[SET][jt][i] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 a = {xd[4 * i], xd[4 * i + 1], xd[4 * i + 2], xd[4 * i + 3]};
#pragma unroll
        for (int jt = 0; jt < C::RTILES; ++jt)
          acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, lb[SET][jt][i]),
                                                            acc[jt], 0, 0, 0);
      }
    }
    // scales: staged [block 0..7 of the span][16 rows] in this wave's LDS;
    // lanes 0..7 keep one 16-byte row each for the store
#pragma unroll
    for (int b = 0; b < 2; ++b) sc_stage[(2 * g + b) * C::ROWS + r] = uint8_t(sb[b]);
    wait_vm_lgkm0<63>();
    if (lane < 8) scv = *reinterpret_cast<const u32x4*>(sc_stage + lane * C::ROWS);
    wait_vm_lgkm0<63>();                                      // staging read done before the next span's writes
    prev_span = span;
  };
  int j0 = 0;
  for (; j0 + C::NSETS <= nmine; j0 += C::NSETS)
    static_for<0, C::NSETS>([&]<int S>() __attribute__((always_inline)) { one_span.template operator()<S>(j0 + S); });
  static_for<0, C::NSETS - 1>([&]<int S>() __attribute__((always_inline)) {
    if (j0 + S < nmine) one_span.template operator()<S>(j0 + S);
  });
  if (prev_span >= 0) store_span();                           // S(last)
  wait_vm_lgkm0<0>();                                         // drain the DMAs past the last span
  // Every lora_down register set stays allocated until here: a set loaded
  // for a span past the wave's last is never read, and without this use the
  // compiler could hand its registers to other values while the (untracked)
  // load is still in flight.
  if constexpr (C::RTILES > 0) {
#pragma unroll
    for (int q = 0; q < C::NSETS; ++q)
#pragma unroll
      for (int jt = 0; jt < LT; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(lb[q][jt][i]));
  }

  if constexpr (C::RTILES > 0) {
    // partial sums of the waves through the drained rings: red[wave][jt][lane]
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < C::RTILES; ++jt)
      *reinterpret_cast<f32x4_t*>(smem + ((wave * C::RTILES + jt) * kWave + lane) * 16) = acc[jt];
    __syncthreads();
    // wave w finishes rank tiles w, w + WAVES, ...: lane (col, g) holds rows
    // 4g .. 4g+3 of rank 16 jt + col
    for (int jt = wave; jt < C::RTILES; jt += C::WAVES) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < C::WAVES; ++w)
        s += *reinterpret_cast<const f32x4_t*>(smem + ((w * C::RTILES + jt) * kWave + lane) * 16);
      const int rank = 16 * jt + (lane & 15);
      if (rank < R) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + 4 * g + e;
          if (row < M) {
            const __bf16 v = __bf16(s[e]);   // round to nearest even
            p.lora_act_in[uint32_t(row) * uint32_t(R) + uint32_t(rank)] = __builtin_bit_cast(uint16_t, v);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side

struct ProdVariant {
  const void* kernel;
  int waves, rtiles, lds;
};

template <int WAVES, int RTILES>
ProdVariant prod_variant() {
  using C = ProdCfg<WAVES, RTILES>;
  return ProdVariant{reinterpret_cast<const void*>(producer_kernel<C>), WAVES, RTILES, C::LDS};
}

// By rank: R == 0, R <= 16, R <= 32 with 8 waves per 16 rows; R == 0 and
// R <= 16 also with 16 waves, for when M / 16 workgroups would leave compute
// units idle (at R <= 32 sixteen waves' registers would spill); R <= 128 with
// 4 waves (its double-buffered lora_down operands need the register file of
// one wave per SIMD).
static const ProdVariant kProdVariants[] = {prod_variant<8, 0>(),  prod_variant<8, 1>(), prod_variant<8, 2>(),
                                            prod_variant<16, 0>(), prod_variant<16, 1>(), prod_variant<4, 8>()};

static int prod_variant_index(int M, int R) {
  if (R > 32) return 5;
  const int rank = R == 0 ? 0 : R <= 16 ? 1 : 2;
  const bool few_rows = (M + 15) / 16 < 192;
  return few_rows && rank < 2 ? 3 + rank : rank;
}

}  // namespace w4a4

using namespace w4a4;

extern "C" int quantize_w4a4_act(const uint16_t* x, const uint16_t* lora_down, uint8_t* act,
                                 uint8_t* ascales, uint16_t* lora_act_in, int M, int K, int R,
                                 void* stream) {
  if (!(M >= 1 && K >= 16 && K % 16 == 0 && R >= 0 && R <= QUANTIZE_W4A4_MAX_R)) return GEMM_W4A4_EINVAL;
  const int64_t lim = int64_t(1) << 31;
  if (int64_t(M) * K * 2 >= lim || int64_t(R) * K * 2 >= lim || int64_t(M) * R * 2 >= lim)
    return GEMM_W4A4_EINVAL;
  if (!x || !act || !ascales || (R > 0 && (!lora_down || !lora_act_in))) return GEMM_W4A4_EINVAL;
  if ((uintptr_t(x) | (R > 0 ? uintptr_t(lora_down) : 0u)) & 15u) return GEMM_W4A4_EALIGN;
  if ((uintptr_t(act) & 7u) || (R > 0 && (uintptr_t(lora_act_in) & 1u))) return GEMM_W4A4_EALIGN;
  const size_t Ms = size_t(M), Ks = size_t(K), Rs = size_t(R);
  const struct { const void* p; size_t n; } outs[] = {
      {act, Ms * Ks / 2}, {ascales, Ks / 16 * Ms}, {lora_act_in, R > 0 ? Ms * Rs * 2 : 0}};
  const struct { const void* p; size_t n; } ins[] = {{x, Ms * Ks * 2}, {lora_down, Rs * Ks * 2}};
  for (int a = 0; a < 3; ++a) {
    for (const auto& in : ins)
      if (overlaps(outs[a].p, outs[a].n, in.p, in.n)) return GEMM_W4A4_EOVERLAP;
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return GEMM_W4A4_EOVERLAP;
  }
  const int dev_rc = check_device();
  if (dev_rc != GEMM_W4A4_OK) return dev_rc;
  const ProdVariant& v = kProdVariants[prod_variant_index(M, R)];
  ProdParams prm{x, lora_down, act, ascales, lora_act_in, M, K, R};
  void* args[] = {&prm};
  const hipError_t e = hipLaunchKernel(v.kernel, dim3((M + 15) / 16), dim3(v.waves * kWave), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}
