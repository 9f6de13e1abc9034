// w4a4_producer.hip — the memory-bound half of SVDQuant W4A4 for gfx950: the
// bf16 activations x [M, K] quantised to the fused GEMM's NVFP4 operand (act
// [M, K/2], two E2M1 codes a byte, low nibble = even k; ascales [K/16, M], one
// FP8-E4M3 scale per 16 k) and the LoRA-down product lora_act_in [M, R] =
// x @ lora_down^T with lora_down [R, K]. The SVDQuant W4A4 on Blackwell page
// calls the GEMM the compute-bound half (section 1) and fixes these layouts
// (sections 2 and 3.1); the scale and rounding rule is this library's
// reading, stated in gemm_w4a4.h.
//
// Design (one workgroup of 4 waves per ROWS = 16 * RT rows of x):
//  * x is read once. The workgroup's rows are cut into spans of 128 k; wave w
//    takes spans w, w+4, w+8, ... and streams them through a private LDS ring
//    (DEPTH spans, 32 KiB) by direct-to-LDS DMA, so the loop needs no
//    workgroup barrier. Each 256-byte row of a span is stored with its 16-byte
//    chunks XOR-swizzled by row, so that the reads below hit distinct banks.
//  * Lane (r, g) holds row r (of each 16-row tile), k = 32g .. 32g+31 of the
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

// RT row tiles of 16 per workgroup, RTILES rank tiles of 16 (R <= 16 * RTILES).
template <int RT_, int RTILES_>
struct ProdCfg {
  static constexpr int RT = RT_, RTILES = RTILES_;
  static constexpr int WAVES = 4, THREADS = WAVES * kWave;
  static constexpr int ROWS = 16 * RT;
  static constexpr int SPAN_K = 128;
  static constexpr int TILE_BYTES = 16 * SPAN_K * 2;            // one 16-row tile of a span (4 KiB)
  static constexpr int SPAN_BYTES = RT * TILE_BYTES;
  static constexpr int DEPTH = 32768 / SPAN_BYTES;                // spans in flight per wave
  static constexpr int RING = DEPTH * SPAN_BYTES;                 // per wave
  static constexpr int SC_BYTES = 8 * ROWS;                       // staged scale bytes of a span
  static constexpr int SC_OFF = WAVES * RING;
  static constexpr int RED_BYTES = WAVES * RT * RTILES * kWave * 16;   // end-of-loop partial sums
  static constexpr int LDS = SC_OFF + WAVES * SC_BYTES;
  static constexpr int DMA_PER_SPAN = SPAN_BYTES / (kWave * 16);  // 16-byte DMA rounds per span
  static constexpr int VM_AFTER = (DEPTH - 1) * DMA_PER_SPAN;     // DMA rounds younger than a span's
  static_assert(DEPTH >= 2 && VM_AFTER < 64, "ring depth");
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
// arithmetic on the float32 bits: subnormals below 2^-6 on the 2^-9 grid).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  if (v < 0.015625f) {   // 2^-6: subnormal grid m * 2^-9, m = 0 .. 8 (8 is the first normal)
    const float q = v * 512.0f + 8388608.0f;   // 2^23: adding it rounds to an integer, ties to even
    return __builtin_bit_cast(uint32_t, q) - 0x4B000000u;
  }
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);   // round the mantissa to 3 bits, ties to even
  return ((r >> 20) - (120u << 3)) & 0xFFu;             // exponent bias 127 -> 7, mantissa 3 bits
}

// Value of an E4M3FN byte b in 0x00 .. 0x7E.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  if (b < 8u) return float(b) * 0.001953125f;   // m * 2^-9
  return __builtin_bit_cast(float, ((b + (120u << 3)) << 20));
}

// One 16-value block (8 dwords of bf16 pairs) -> its scale byte and the 16
// codes packed as two dwords (low nibble first). Exact decisions:
//  * amax / 6 is divided correctly rounded; the float32 quotient lies on the
//    same side of every E4M3 midpoint as the exact one (ties are exact in
//    float32, other quotients are at least 2^-13 relative away), and the
//    integer rounding above is exact.
//  * |x| / s: within 2^-22 relative of the exact quotient, which is either
//    exactly an E2M1 midpoint (a multiple of 0.25) or at least 2^-10 away from
//    every one; snapping to the 2^-12 grid (adding and subtracting 2048)
//    restores the exact midpoints and keeps every other quotient on its side,
//    so the conversion's nearest-even rounding decides like the exact one.
__device__ __forceinline__ void quantize_block(const uint32_t (&d)[8], uint32_t& sbyte, uint32_t& lo,
                                               uint32_t& hi) {
  // |x| bit patterns order like the magnitudes (NaN above infinity above
  // every finite value): a packed 16-bit max over the pairs, then the halves
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, d[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[i] & 0x7FFF7FFFu));
  const uint32_t amax_bits = max(uint32_t(m[0]), uint32_t(m[1]));
  if (amax_bits >= 0x7F80u) {   // NaN or infinity in the block
    sbyte = 0x7Fu;
    lo = hi = 0u;
    return;
  }
  const float amax = __builtin_bit_cast(float, amax_bits << 16);
  const uint32_t sb = e4m3_rne(fminf(amax / 6.0f, 448.0f));
  const float s = e4m3_value(sb);
  const float r = s > 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
  sbyte = sb;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xl = __builtin_bit_cast(float, d[i] << 16);
    const float xh = __builtin_bit_cast(float, d[i] & 0xFFFF0000u);
    float ql = __builtin_fmaf(__builtin_fabsf(xl), r, 2048.0f) - 2048.0f;
    float qh = __builtin_fmaf(__builtin_fabsf(xh), r, 2048.0f) - 2048.0f;
    ql = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, ql) & 0x7FFFFFFFu) |
                                       (__builtin_bit_cast(uint32_t, xl) & 0x80000000u));
    qh = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, qh) & 0x7FFFFFFFu) |
                                       (__builtin_bit_cast(uint32_t, xh) & 0x80000000u));
    // element 2i is k even (low nibble of byte i), 2i+1 odd; byte i of the 8
    switch (i & 3) {   // byte select must be an immediate; folds after unrolling
      case 0: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], ql, qh, 1.0f, 0); break;
      case 1: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], ql, qh, 1.0f, 1); break;
      case 2: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], ql, qh, 1.0f, 2); break;
      default: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], ql, qh, 1.0f, 3); break;
    }
  }
  lo = w[0];
  hi = w[1];
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

  // DMA of this wave's j-th span into ring slot j % DEPTH. Round u of tile t:
  // lane l writes slot position (row 4u + l/16, chunk l%16) and reads data
  // chunk (l%16) ^ row of that row. Spans past the wave's last one re-read it
  // (never consumed); k past K and rows past M read clamped in-range bytes.
  auto dma_span = [&](int j) __attribute__((always_inline)) {
    const int jj = nmine > 0 ? min(j, nmine - 1) : 0;
    const int span = wave_u + C::WAVES * jj;
    uint8_t* slot = ring + (j % C::DEPTH) * C::SPAN_BYTES;
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int lr = 4 * u + (lane >> 4);                       // row inside the tile
        const int row = min(m0 + 16 * t + lr, M - 1);
        const int chunk = (lane & 15) ^ lr;                       // 16-byte chunk = 8 k
        const int kk = span * C::SPAN_K + 8 * chunk;
        const uint32_t kb = kk < K ? uint32_t(kk) * 2u : 0u;
        dma<16>(reinterpret_cast<const uint8_t*>(p.x) + uint32_t(row) * row_bytes + kb,
                slot + t * C::TILE_BYTES + u * 1024);
      }
  };

  f32x4_t acc[C::RT][C::RTILES > 0 ? C::RTILES : 1];
#pragma unroll
  for (int t = 0; t < C::RT; ++t)
#pragma unroll
    for (int j = 0; j < (C::RTILES > 0 ? C::RTILES : 1); ++j) acc[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < C::DEPTH; ++j) dma_span(j);

  const bool act16 = (K & 31) == 0 && (reinterpret_cast<uintptr_t>(p.act) & 15u) == 0;
  const bool sc16 = (M & 15) == 0 && (reinterpret_cast<uintptr_t>(p.ascales) & 15u) == 0;
  uint8_t* sc_stage = smem + C::SC_OFF + wave_u * C::SC_BYTES;

  // Issue order per span j: LoRA-down loads L(j), the LDS reads of span j,
  // the refill DMA(j + DEPTH) of its slot, the stores. Vector-memory ops
  // complete in issue order, so: at the top, DMA(j) is complete once at most
  // the (DEPTH-1) younger DMA groups may be outstanding (any younger loads or
  // stores only make that wait stricter); L(j) is complete once at most the
  // one DMA group issued after it may be.
  for (int j = 0; j < nmine; ++j) {
    const int span = wave_u + C::WAVES * j;
    const int k0 = span * C::SPAN_K + 32 * g;                 // this lane's first k
    wait_vm_lgkm0<C::VM_AFTER>();                             // DMA(j) has landed

    // LoRA-down operands of this span (B: lora_down[rank][k0 + 8i .. +7]);
    // ranks past R re-read rank R-1 (their sums are not stored); k past K
    // re-reads the row's last 8 and is zeroed before use
    u32x4 lb[C::RTILES > 0 ? C::RTILES : 1][4];
    if constexpr (C::RTILES > 0) {
#pragma unroll
      for (int jt = 0; jt < C::RTILES; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rank = min(16 * jt + r, R - 1);
          const int kk = min(k0 + 8 * i, K - 8);
          lb[jt][i] = *reinterpret_cast<const u32x4*>(p.lora_down + uint32_t(rank) * uint32_t(K) + uint32_t(kk));
        }
    }

    const uint8_t* slot = ring + (j % C::DEPTH) * C::SPAN_BYTES;
    uint32_t xd[C::RT][16];
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(slot + t * C::TILE_BYTES + r * 256 +
                                                        (((4 * g + i) ^ r) << 4));
        xd[t][4 * i] = v.x;
        xd[t][4 * i + 1] = v.y;
        xd[t][4 * i + 2] = v.z;
        xd[t][4 * i + 3] = v.w;
      }
    wait_vm_lgkm0<63>();                                      // the slot is read: refill it
    dma_span(j + C::DEPTH);
    // blocks of this lane past K: zero (they add nothing to the LoRA sums and are not stored)
    const bool blk_ok[2] = {k0 < K, k0 + 16 < K};
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!blk_ok[i >> 3]) xd[t][i] = 0u;

    // quantise the lane's two blocks of each row tile
    uint32_t sb[C::RT][2], code[C::RT][4];
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = xd[t][8 * b + i];
        quantize_block(d, sb[t][b], code[t][2 * b], code[t][2 * b + 1]);
      }

    if constexpr (C::RTILES > 0) {
      wait_vm<C::DMA_PER_SPAN>();                             // L(j); DMA(j + DEPTH) may still fly
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // k past K: a zero operand (a NaN weight there must not reach valid sums)
        const bool kin = k0 + 8 * i < K;
#pragma unroll
        for (int t = 0; t < C::RT; ++t) {
          const u32x4 a = {xd[t][4 * i], xd[t][4 * i + 1], xd[t][4 * i + 2], xd[t][4 * i + 3]};
#pragma unroll
          for (int jt = 0; jt < C::RTILES; ++jt) {
            const u32x4 b = kin ? lb[jt][i] : u32x4{0u, 0u, 0u, 0u};
            acc[t][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, b),
                                                                 acc[t][jt], 0, 0, 0);
          }
        }
      }
    }

    // act: 16 bytes (32 codes) per lane and row tile at act[row][k0/2 ..]
#pragma unroll
    for (int t = 0; t < C::RT; ++t) {
      const int row = m0 + 16 * t + r;
      if (row < M) {
        uint8_t* dst = p.act + uint32_t(row) * uint32_t(K / 2) + uint32_t(k0 / 2);
        if (act16 && blk_ok[1]) {
          *reinterpret_cast<u32x4*>(dst) = u32x4{code[t][0], code[t][1], code[t][2], code[t][3]};
        } else {
          if (blk_ok[0]) *reinterpret_cast<u32x2*>(dst) = u32x2{code[t][0], code[t][1]};
          if (blk_ok[1]) *reinterpret_cast<u32x2*>(dst + 8) = u32x2{code[t][2], code[t][3]};
        }
      }
    }
    // scales: staged [block 0..7 of the span][ROWS] in this wave's LDS, then
    // written as rows of ascales
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int b = 0; b < 2; ++b) sc_stage[(2 * g + b) * C::ROWS + 16 * t + r] = uint8_t(sb[t][b]);
    wait_vm_lgkm0<63>();
    constexpr int PIECES = 8 * C::ROWS / 16;                  // 16-byte pieces of the staged scales
    const int kb0 = span * (C::SPAN_K / 16);
    if (lane < PIECES) {
      const int blk = lane / C::RT, part = lane % C::RT;
      const int kb = kb0 + blk, mrow = m0 + 16 * part;
      if (kb < K / 16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sc_stage + blk * C::ROWS + 16 * part);
        uint8_t* dst = p.ascales + uint32_t(kb) * uint32_t(M) + uint32_t(mrow);
        if (sc16 && mrow + 16 <= M) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (mrow + e < M) dst[e] = uint8_t(w4[e >> 2] >> (8 * (e & 3)));
        }
      }
    }
    wait_vm_lgkm0<63>();                                      // staging reads done before the next span's writes
  }
  wait_vm_lgkm0<0>();                                         // drain the DMAs past the last span

  if constexpr (C::RTILES > 0) {
    // partial sums of the four waves through the drained rings:
    // red[wave][t][jt][lane] (16 bytes each)
    __syncthreads();
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int jt = 0; jt < C::RTILES; ++jt)
        *reinterpret_cast<f32x4_t*>(smem + (((wave * C::RT + t) * C::RTILES + jt) * kWave + lane) * 16) =
            acc[t][jt];
    __syncthreads();
    // wave w finishes the (t, jt) pairs with (t * RTILES + jt) % 4 == w:
    // lane (col, g) holds rows 4g .. 4g+3 of rank 16 jt + col
    for (int q = wave; q < C::RT * C::RTILES; q += C::WAVES) {
      const int t = q / C::RTILES, jt = q % C::RTILES;
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < C::WAVES; ++w)
        s += *reinterpret_cast<const f32x4_t*>(smem + (((w * C::RT + t) * C::RTILES + jt) * kWave + lane) * 16);
      const int rank = 16 * jt + (lane & 15);
      if (rank < R) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + 16 * t + 4 * g + e;
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
  int rt, rtiles, rows, lds;
};

template <int RT, int RTILES>
ProdVariant prod_variant() {
  using C = ProdCfg<RT, RTILES>;
  return ProdVariant{reinterpret_cast<const void*>(producer_kernel<C>), RT, RTILES, C::ROWS, C::LDS};
}

// by rank: R == 0, R <= 16, R <= 32, R <= 128; two rows tiles per workgroup
// for the largest ranks, where each workgroup reads all of lora_down once
static const ProdVariant kProdVariants[] = {prod_variant<1, 0>(), prod_variant<1, 1>(), prod_variant<1, 2>(),
                                            prod_variant<2, 8>()};

static int prod_variant_index(int R) { return R == 0 ? 0 : R <= 16 ? 1 : R <= 32 ? 2 : 3; }

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
  const ProdVariant& v = kProdVariants[prod_variant_index(R)];
  ProdParams prm{x, lora_down, act, ascales, lora_act_in, M, K, R};
  void* args[] = {&prm};
  const hipError_t e = hipLaunchKernel(v.kernel, dim3((M + v.rows - 1) / v.rows), dim3(256), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}
