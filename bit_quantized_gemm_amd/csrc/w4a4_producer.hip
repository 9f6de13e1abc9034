// w4a4_producer.hip — the memory-bound half of SVDQuant W4A4 for gfx950: the
// bf16 activations x [M, K] quantised to the fused GEMM's NVFP4 operand (act
// [M, K/2], two E2M1 codes a byte, low nibble = even k; ascales [K/16, M], one
// FP8-E4M3 scale per 16 k) and the LoRA-down product lora_act_in [M, R] =
// x @ lora_down^T with lora_down [R, K]. The SVDQuant W4A4 on Blackwell page
// calls the GEMM the compute-bound half (section 1) and fixes these layouts
// (sections 2 and 3.1); the scale and rounding rule is this library's
// reading, stated in gemm_w4a4.h.
//
// Design. Ranks 0 < R <= 32 run a narrow kernel: one workgroup of 8 waves per
// 16 rows of x and one slice of K.
//  * x is read once. K is cut into spans of 128; a workgroup takes the spans
//    of its K slice, wave w the spans w, w+WAVES, ... of them, streamed through a
//    private LDS ring of DEPTH slots by direct-to-LDS DMA, so the loop needs
//    no workgroup barrier. Each 256-byte row of a span is stored with its
//    16-byte chunks XOR-swizzled by row, so that the reads below hit distinct
//    banks. Loads are buffer loads: a per-lane offset fixed for the whole
//    kernel into a descriptor of the span's base and the tensor's remaining
//    bytes, in scalar registers. Reads past the tensor's end return zeros and
//    reads past K in the span that crosses it land in the next row, zeroed at
//    use, so no address is clamped.
//  * When the row blocks (M / 16) do not fill the chip, K is split into
//    slices over several workgroups: each writes its float32 LoRA partial
//    sums to a scratch buffer, and the last of them to finish (a counter per
//    row block) adds the slices in slice order and writes lora_act_in, so
//    the result does not depend on the order the workgroups ran in.
// Ranks R > 32, and R = 0, run the wide kernel (producer_wide_kernel): four
// waves share 128 rows, each streaming its own 32 rows of x, while the span's
// lora_down tile is DMA'd once per workgroup into a shared LDS ring; its K
// slices' partial sums are added by a second launch (producer_reduce_kernel).
//  * Lane (r, g) holds row r, k = 32g .. 32g+31 of the span: two whole
//    16-value blocks, so a block's amax needs no cross-lane step. Scale and
//    codes are decided exactly (see quantize_block), codes are packed by the
//    FP4 conversion, act is written as 16 (or 2 x 8) bytes per lane and the
//    scale bytes are gathered through LDS into 16-byte rows of ascales.
//  * The same registers are the A operand of v_mfma_f32_16x16x32_bf16: in
//    k-step i lane (r, g) supplies x[r][32g + 8i .. +7] and, as B operand,
//    lora_down[rank][32g + 8i .. +7] (any k order works if both sides agree).
//    The waves' partial sums meet once through LDS at the end.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "gemm_w4a4.h"
#include "w4a4_common.hpp"
#include "w4a4_host.hpp"

namespace w4a4 {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// WAVES waves per workgroup, RTILES rank tiles of 16 (1 or 2: 0 < R <= 16 *
// RTILES), DEPTH ring slots per wave.
template <int WAVES_, int RTILES_, int DEPTH_>
struct ProdCfg {
  static constexpr int WAVES = WAVES_, RTILES = RTILES_, DEPTH = DEPTH_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int ROWS = 16;
  static constexpr int SPAN_K = 128;
  static constexpr int SPAN_BYTES = ROWS * SPAN_K * 2;            // one span of 16 rows (4 KiB)
  static constexpr int RING = DEPTH * SPAN_BYTES;                 // per wave
  static constexpr int SC_BYTES = 8 * ROWS;                       // staged scale bytes of a span
  static constexpr int SC_OFF = WAVES * RING;
  static constexpr int RED_BYTES = WAVES * RTILES * kWave * 16;   // end-of-loop partial sums
  static constexpr int LDS = SC_OFF + WAVES * SC_BYTES;
  static constexpr int D = SPAN_BYTES / (kWave * 16);             // 16-byte DMA rounds per span
  static constexpr int NL = 4 * RTILES;                           // lora_down loads per span
  // lora_down operands of a span, L(j), go to register set j % 2: L(j+1) is
  // issued early in span j, beside the refill DMA(j + DEPTH).
  static constexpr int NSETS = 2;
  // Issue order: DMA(0), L(0), DMA(1); then per span j the stores S(j-1) of
  // the previous span's results and the pair L(j+1), DMA(j+2). A pair past
  // the wave's last span is issued as the same loads on an empty descriptor
  // (they read nothing), so that every count below is the same in every
  // span. Loads complete in issue order and a store can only make a count of
  // loads stricter, so waiting until at most X vector-memory ops remain
  // completes every load with at least X younger loads:
  //   DMA(j): one younger pair (DMA(0): L(0) and DMA(1), waited for by the
  //           prologue itself);
  //   L(j):   DMA(j+1) and span j's pair.
  static constexpr int VM_X = D + NL;
  static constexpr int VM_X0 = D + NL;
  static constexpr int VM_L = 2 * D + NL;
  static_assert(RTILES >= 1 && RTILES <= 2, "0 < R <= 32: R = 0 and larger ranks run the wide kernel");
  static_assert(DEPTH == 2, "the wait counts above are those of a two-slot ring");
  static_assert(VM_L < 64, "vmcnt range");
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
  int ks, sps;          // K slices per row block, spans per slice
  float* part;          // ks > 1 and R > 0: float32 partial sums, [row block][slice][rank][16 rows]
                        // (narrow kernels) or [row block][slice][128 rows][rank] (wide kernel)
  uint32_t* count;      // ks > 1 and R > 0: arrivals per row block, zero between calls
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
//    2^-9 relative from every E4M3 midpoint; the integer rounding above is
//    exact.
//  * x / s: P = x * (4096 / s), with 4096 / s from the reciprocal, is within
//    2^-21 relative of 4096 x / s. For |x| / s <= 6.5 that exact quotient is
//    either exactly an E2M1 midpoint (a multiple of 1024) or at least 4 away
//    from every one, so rounding P to an integer (nearest even) gives the
//    midpoints exactly and keeps every other quotient on its side. The FP4
//    conversion divides by its scale's power of two (4096) exactly and rounds
//    to nearest even, so it decides like the exact quotient; larger
//    quotients saturate either way. The rounding keeps the sign of zero, and
//    an infinite P converts to the largest code.
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
  const float c = s > 0.0f ? __builtin_amdgcn_rcpf(s) * 4096.0f : 0.0f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // element 2i (k even) is the low half of the dword: low nibble of byte i
    const float pl = __builtin_rintf(__builtin_bit_cast(float, d[i] << 16) * c);
    const float ph = __builtin_rintf(__builtin_bit_cast(float, d[i] & 0xFFFF0000u) * c);
    switch (i & 3) {   // byte select must be an immediate; folds after unrolling
      case 0: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], pl, ph, 4096.0f, 0); break;
      case 1: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], pl, ph, 4096.0f, 1); break;
      case 2: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], pl, ph, 4096.0f, 2); break;
      default: w[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[i >> 2], pl, ph, 4096.0f, 3); break;
    }
  }
  sbyte = finite ? sb : 0x7Fu;
  lo = finite ? w[0] : 0u;
  hi = finite ? w[1] : 0u;
}

// Raw buffer descriptor of `bytes` bytes from `base` (gfx9 format word),
// in scalar registers (the values are wave-uniform; readfirstlane says so
// where the compiler cannot prove it).
__device__ __forceinline__ u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a))),
               uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xFFFFu)),
               uint32_t(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000u};
}

// 16-byte buffer load the compiler does not track (see load_lora): per-lane
// offset + immediate into the descriptor's range (zeros past its end).
template <int IMM>
__device__ __forceinline__ void load_untracked(u32x4& dst, uint32_t voff, const u32x4& desc) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3"
               : "=v"(dst) : "v"(voff), "s"(desc), "i"(IMM) : "memory");
}

// The same descriptor for the buffer builtins.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Direct-to-LDS 16-byte buffer load: lane l writes lds + 16 l.
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Split-K partial sums: float32, [row block][slice][rank][ROWS rows], so
// that the four rows an MFMA lane holds for one rank are one 16-byte piece
// (in the narrow kernels stored and loaded as two 8-byte device-scope atomic
// accesses).
constexpr int kProdMaxSlices = 8;        // narrow kernels: one register per slice and group
constexpr int kProdMaxWideSlices = 64;   // the wide kernel (a second launch adds them)

// (The whole vector is reinterpreted: this compiler's bit-cast of a single
// vector element reads the vector's first element.)
__device__ __forceinline__ void store_partial4(float* dst, const f32x4_t& v) {
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  const u64x2 w = __builtin_bit_cast(u64x2, v);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
  __hip_atomic_store(d, uint64_t(w.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, uint64_t(w.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K split over the narrow kernels' workgroups: the last workgroup of row
// block rb (rows m0 .. m0+ROWS-1) to finish adds the slices' partial sums in
// slice order and writes lora_act_in (16 rows: at most 4R groups, one per
// thread). The partial sums and the counter are device-scope atomic
// accesses, each coherent across the compute dies by itself; every wave
// waits until its stores are acknowledged before the barrier, which orders
// the sums before the count, so no cache write-back or invalidation is
// needed. Every slice's loads are issued before they are added. `flag` is
// one word of free LDS.
template <int ROWS, int THREADS>
__device__ __forceinline__ void finish_split(const ProdParams& p, int rb, int m0, uint32_t* flag) {
  constexpr int GR = 1;
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(p.count + rb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            uint32_t(p.ks - 1);
  __syncthreads();
  if (*flag) {
    const int R = p.R, ks = p.ks;
    const int ng = (ROWS / 4) * R;   // groups of four rows of one rank, per slice
    const uint64_t* base = reinterpret_cast<const uint64_t*>(p.part + uint32_t(rb) * uint32_t(ks) * uint32_t(ROWS * R));
    for (int g0 = threadIdx.x; g0 < ng; g0 += GR * THREADS) {
      uint64_t v[GR][kProdMaxSlices][2];
#pragma unroll
      for (int u = 0; u < GR; ++u) {
        const int gi = g0 + u * THREADS;
#pragma unroll
        for (int q = 0; q < kProdMaxSlices; ++q)
          if (q < ks && gi < ng) {
            const uint64_t* src = base + 2 * (uint32_t(q) * uint32_t(ng) + uint32_t(gi));
            v[u][q][0] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v[u][q][1] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
      }
#pragma unroll
      for (int u = 0; u < GR; ++u) {
        const int gi = g0 + u * THREADS;
        if (gi >= ng) continue;
        float sm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < kProdMaxSlices; ++q)
          if (q < ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm[e] += __builtin_bit_cast(float, uint32_t(v[u][q][e >> 1] >> (32 * (e & 1))));
        const int rank = gi / (ROWS / 4), row = m0 + 4 * (gi % (ROWS / 4));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row + e < p.M) {
            const __bf16 b = __bf16(sm[e]);   // round to nearest even
            p.lora_act_in[uint32_t(row + e) * uint32_t(R) + uint32_t(rank)] = __builtin_bit_cast(uint16_t, b);
          }
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(p.count + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
  const int rb = blockIdx.x / p.ks, z = blockIdx.x - rb * p.ks;
  const int m0 = rb * C::ROWS;
  const int nsp = (K + C::SPAN_K - 1) / C::SPAN_K;
  const int s_end = min(nsp, (z + 1) * p.sps);
  const int first = z * p.sps + wave_u;                                  // this wave's first span
  const int n = first < s_end ? (s_end - 1 - first) / C::WAVES + 1 : 0;   // and its number of spans
  const int tail_span = (K % C::SPAN_K) != 0 ? nsp - 1 : -1;             // the span crossing K
  const uint32_t row_bytes = uint32_t(K) * 2u;
  uint8_t* ring = smem + wave_u * C::RING;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.x);

  // DMA round u of a span: lane l writes slot position (row 4u + l/16, chunk
  // l%16) and reads data chunk (l%16) ^ row of that row; rows past M read
  // row M-1 (never stored).
  const uint32_t x_bytes = uint32_t(M) * row_bytes;
  uint32_t xoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int lr = 4 * u + g;
    xoff[u] = uint32_t(min(m0 + lr, M - 1)) * row_bytes + uint32_t((r ^ lr) << 4);
  }
  // span j of this wave into slot j % DEPTH; j >= n: a dummy of the same
  // shape on an empty descriptor (reads nothing, writes zeros to the slot,
  // which holds no span still to be read)
  auto dma_span = [&](int j) __attribute__((always_inline)) {
    const bool valid = j < n;
    const uint32_t sb = valid ? uint32_t(first + C::WAVES * j) * uint32_t(C::SPAN_K * 2) : 0u;
    const __amdgpu_buffer_rsrc_t desc = buffer_rsrc(xb + sb, valid ? x_bytes - sb : 0u);
    uint8_t* slot = ring + (j % C::DEPTH) * C::SPAN_BYTES;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_buf(desc, xoff[u], slot + u * 1024);
  };

  f32x4_t acc[C::RTILES];
#pragma unroll
  for (int jt = 0; jt < C::RTILES; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LoRA-down operands of this wave's j-th span into a register set (B:
  // lora_down[rank][k0 + 8i .. +7]); ranks past R re-read rank R-1 (their
  // sums are not stored), and in the span crossing K, k past K reads the next
  // rank's values or zeros (zeroed at use).
  //
  // Issued as explicit buffer_load_dwordx4, which the compiler does not
  // track: with stores in flight it would otherwise wait for every
  // outstanding vector-memory op (vmcnt(0)) before the first use, the ring's
  // DMAs included. The explicit waits count loads only, and scheduling fences
  // keep every use after its wait.
  constexpr int LT = C::RTILES;
  u32x4 lb[C::NSETS][LT][4];
  uint32_t loff[LT];
#pragma unroll
  for (int jt = 0; jt < LT; ++jt)
    loff[jt] = uint32_t(min(16 * jt + r, R - 1)) * row_bytes + uint32_t(64 * g);
  const uint8_t* ldb = reinterpret_cast<const uint8_t*>(p.lora_down);
  const uint32_t ld_bytes = uint32_t(R) * row_bytes;
  // span j; j >= n: a dummy on an empty descriptor (reads nothing; the set
  // is not used)
  auto load_lora = [&](u32x4 (&dst)[LT][4], int j) __attribute__((always_inline)) {
    const bool valid = j < n;
    const uint32_t sb = valid ? uint32_t(first + C::WAVES * j) * uint32_t(C::SPAN_K * 2) : 0u;
    const u32x4 desc = buffer_desc(ldb + sb, valid ? ld_bytes - sb : 0u);
#pragma unroll
    for (int jt = 0; jt < LT; ++jt) {
      const uint32_t off = loff[jt];
      load_untracked<0>(dst[jt][0], off, desc);
      load_untracked<16>(dst[jt][1], off, desc);
      load_untracked<32>(dst[jt][2], off, desc);
      load_untracked<48>(dst[jt][3], off, desc);
    }
  };
  // the pair of span t: L(t+1), DMA(t+DEPTH)
  auto issue_pair = [&]<int NEXT_SET>(int t) __attribute__((always_inline)) {
    load_lora(lb[NEXT_SET], t + 1);
    dma_span(t + C::DEPTH);
  };

  // prologue: DMA(0 .. DEPTH-2), L(0), DMA(DEPTH-1)
#pragma unroll
  for (int t = 0; t < C::DEPTH - 1; ++t) dma_span(t);
  load_lora(lb[0], 0);
  dma_span(C::DEPTH - 1);
  wait_vm_lgkm0<C::VM_X0>();   // DMA(0): its count differs from the loop's

  // output addresses: act row m0 + r from k0 / 2; ascales row (block) lane
  // of the span, 16 consecutive m
  const bool row_ok = m0 + r < M;
  const uint32_t aoff = uint32_t(min(m0 + r, M - 1)) * uint32_t(K / 2) + uint32_t(16 * g);
  const uint32_t soff = uint32_t(lane & 7) * uint32_t(M) + uint32_t(m0);
  const bool act16 = (K & 31) == 0 && (reinterpret_cast<uintptr_t>(p.act) & 15u) == 0;
  // widest store a scale row allows: rows of ascales are M bytes apart
  const uintptr_t sc_align = reinterpret_cast<uintptr_t>(p.ascales) | uintptr_t(M);
  const int sc_w = (sc_align & 15u) == 0 ? 16 : (sc_align & 7u) == 0 ? 8 : (sc_align & 3u) == 0 ? 4 : 1;
  uint8_t* sc_stage = smem + C::SC_OFF + wave_u * C::SC_BYTES;

  // The results of a span are stored at the start of the next one, before its
  // pair of loads, so that no store lies between a load and the ops its
  // wait counts.
  uint32_t code[4] = {0u, 0u, 0u, 0u};   // the previous span's 32 codes of this lane
  u32x4 scv = {0u, 0u, 0u, 0u};          // lanes 0..7: one 16-byte row of its scales
  const int nv = min(C::ROWS, M - m0);   // valid rows of the block
  auto store_span = [&](int span) __attribute__((always_inline)) {
    uint8_t* abase = p.act + uint32_t(span) * uint32_t(C::SPAN_K / 2);
    uint8_t* sbase = p.ascales + uint32_t(span) * uint32_t(C::SPAN_K / 16) * uint32_t(M);
    const bool tail = span == tail_span;
    const int k0 = span * C::SPAN_K + 32 * g;
    if (row_ok) {
      if (act16 && !tail) {
        *reinterpret_cast<u32x4*>(abase + aoff) = u32x4{code[0], code[1], code[2], code[3]};
      } else {
        if (k0 < K) *reinterpret_cast<u32x2*>(abase + aoff) = u32x2{code[0], code[1]};
        if (k0 + 16 < K) *reinterpret_cast<u32x2*>(abase + aoff + 8) = u32x2{code[2], code[3]};
      }
    }
    if (lane < 8 && span * (C::SPAN_K / 16) + lane < K / 16) {
      if (sc_w == 16) {
        *reinterpret_cast<u32x4*>(sbase + soff) = scv;
      } else if (sc_w == 8 && nv == C::ROWS) {
        *reinterpret_cast<u32x2*>(sbase + soff) = u32x2{scv.x, scv.y};
        *reinterpret_cast<u32x2*>(sbase + soff + 8) = u32x2{scv.z, scv.w};
      } else if (sc_w == 4 && nv == C::ROWS) {
        uint32_t* d = reinterpret_cast<uint32_t*>(sbase + soff);
        d[0] = scv.x;
        d[1] = scv.y;
        d[2] = scv.z;
        d[3] = scv.w;
      } else {
        const uint64_t lo = uint64_t(scv.x) | (uint64_t(scv.y) << 32), hi = uint64_t(scv.z) | (uint64_t(scv.w) << 32);
#pragma unroll 1
        for (int e = 0; e < nv; ++e) sbase[soff + e] = uint8_t((e < 8 ? lo : hi) >> (8 * (e & 7)));
      }
    }
  };

  // span j uses lora_down set j % 2; the loop below is unrolled twice
  auto one_span = [&]<int SET>(int j) __attribute__((always_inline)) {
    constexpr int NEXT = (SET + 1) % C::NSETS;
    const int span = first + C::WAVES * j;
    const bool tail = span == tail_span;
    wait_vm_lgkm0<C::VM_X>();                                 // DMA(j) has landed
    // scheduling fences keep the issue order the wait counts rely on
    __builtin_amdgcn_sched_barrier(0);
    if (j > 0) store_span(span - C::WAVES);                   // S(j-1)
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
    wait_vm_lgkm0<63>();                                      // the slot is read
    __builtin_amdgcn_sched_barrier(0);
    issue_pair.template operator()<NEXT>(j);                  // L(j+1), DMA(j+DEPTH)
    __builtin_amdgcn_sched_barrier(0);
    if (tail) {
      // this lane's blocks past K: zero (they add nothing to the LoRA sums
      // and are not stored)
      const int k0 = span * C::SPAN_K + 32 * g;
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
    // scales: staged [block 0..7 of the span][16 rows] in this wave's LDS;
    // lanes 0..7 take one 16-byte row each for the store
#pragma unroll
    for (int b = 0; b < 2; ++b) sc_stage[(2 * g + b) * C::ROWS + r] = uint8_t(sb[b]);

    // the MFMAs of register set Q once its loads landed
    auto lora_mfma = [&]<int Q>() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<C::VM_L>();                                     // L(j)
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");                          // nothing reads lb[Q] before this point
      if (tail) {
        // k past K: a zero operand (a NaN weight there must not reach valid sums)
        const int k0 = span * C::SPAN_K + 32 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jt = 0; jt < LT; ++jt)
            if (k0 + 8 * i >= K) lb[Q][jt][i] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 a = {xd[4 * i], xd[4 * i + 1], xd[4 * i + 2], xd[4 * i + 3]};
#pragma unroll
        for (int jt = 0; jt < LT; ++jt)
          acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, lb[Q][jt][i]), acc[jt], 0, 0, 0);
      }
    };
    lora_mfma.template operator()<SET>();
    wait_vm_lgkm0<63>();
    if (lane < 8) scv = *reinterpret_cast<const u32x4*>(sc_stage + lane * C::ROWS);
    wait_vm_lgkm0<63>();                                      // staging read done before the next span's writes
  };
  int j0 = 0;
  for (; j0 + C::NSETS <= n; j0 += C::NSETS)
    static_for<0, C::NSETS>([&]<int S>() __attribute__((always_inline)) { one_span.template operator()<S>(j0 + S); });
  static_for<0, C::NSETS - 1>([&]<int S>() __attribute__((always_inline)) {
    if (j0 + S < n) one_span.template operator()<S>(j0 + S);
  });
  if (n > 0) store_span(first + C::WAVES * (n - 1));          // S(last)
  wait_vm_lgkm0<0>();                                         // drain the loads past the last span
  // Every lora_down register set stays allocated until here: a set loaded
  // past the wave's last span is never read, and without this use the
  // compiler could hand its registers to other values while the (untracked)
  // load is still in flight.
#pragma unroll
  for (int q = 0; q < C::NSETS; ++q)
#pragma unroll
    for (int jt = 0; jt < LT; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(lb[q][jt][i]));

  // partial sums of the waves through the drained rings: red[wave][jt][lane]
  __syncthreads();
#pragma unroll
  for (int jt = 0; jt < C::RTILES; ++jt)
    *reinterpret_cast<f32x4_t*>(smem + ((wave * C::RTILES + jt) * kWave + lane) * 16) = acc[jt];
  __syncthreads();
  // wave w finishes rank tiles w, w + WAVES, ...: lane (col, g) holds rows
  // 4g .. 4g+3 of rank 16 jt + col
  const bool split = p.ks > 1;
  for (int jt = wave; jt < C::RTILES; jt += C::WAVES) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w)
      s += *reinterpret_cast<const f32x4_t*>(smem + ((w * C::RTILES + jt) * kWave + lane) * 16);
    const int rank = 16 * jt + (lane & 15);
    if (rank < R) {
      if (split) {
        store_partial4(p.part + (uint32_t(blockIdx.x) * uint32_t(R) + uint32_t(rank)) * uint32_t(C::ROWS) +
                           uint32_t(4 * g), s);
      } else {
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
  if (split) finish_split<C::ROWS, C::THREADS>(p, rb, m0, reinterpret_cast<uint32_t*>(smem + C::SC_OFF));
}

// ------------------------------------------------------------------ wide variant
//
// The largest ranks (32 < R <= 128). Read per 16 rows, a span's lora_down
// tile (R x 128 values) outweighs its x by R/16 and its loads touch two
// cache lines per 32 bytes used; here one workgroup of 4 waves takes 128
// rows (32 per wave, two 16-row MFMA tiles sharing each operand) and every
// wave the same span: the span's lora_down tile is brought into LDS once per
// workgroup by direct-to-LDS DMA of whole rows (each wave a quarter of its
// rank rows), and each wave reads its B operands from there. x moves through
// a private ring per wave as in the narrow kernel; K is split over
// workgroups when the row blocks alone do not fill the chip.
template <int RTILES_>
struct WideCfg {
  static constexpr int WAVES = 4, RTILES = RTILES_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int ROWS_W = 32, ROWS = WAVES * ROWS_W;    // rows per wave, per workgroup
  static constexpr int SPAN_K = 128, ROW_SPAN = SPAN_K * 2;  // bytes of one row in a span
  static constexpr int X_SLOT = ROWS_W * ROW_SPAN;           // one span of a wave's rows (8 KiB)
  static constexpr int X_RING = 2 * X_SLOT;                  // per wave
  static constexpr int L_ROWS = 16 * RTILES;                 // rank rows of a lora_down tile
  static constexpr int L_SLOT = L_ROWS * ROW_SPAN;           // one span's tile
  static constexpr int L_OFF = WAVES * X_RING;
  static constexpr int SC_OFF = L_OFF + 2 * L_SLOT;
  static constexpr int SC_BYTES = 2 * 8 * 16;                // staged scales of a span, per wave
  static constexpr int LDS = SC_OFF + WAVES * SC_BYTES;
  static constexpr int DX = X_SLOT / (kWave * 16);           // x DMA rounds per wave and span
  static constexpr int DL = L_SLOT / WAVES / (kWave * 16);   // lora_down DMA rounds per wave and span
  // Issue order: X(0), L(0), X(1); then per span j, after its barrier,
  // L(j+1) and, once the wave has read its x slot, X(j+2). At the start of
  // span j, L(j) (this wave's part) is followed by X(j+1) only, and X(j) is
  // older than L(j): waiting until DX ops remain completes both.
  static constexpr int VM_J = DX;
  static_assert(DX <= 63 && RTILES % 1 == 0, "wait counts");
  static_assert(LDS <= kLdsLimit, "LDS budget");
};

template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void producer_wide_kernel(const ProdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int r = lane & 15, g = lane >> 4;
  const int M = p.M, K = p.K, R = p.R;
  const int rb = blockIdx.x / p.ks, z = blockIdx.x - rb * p.ks;
  const int m0 = rb * C::ROWS;
  const int mw = m0 + wave_u * C::ROWS_W;                                // this wave's first row
  const int nsp = (K + C::SPAN_K - 1) / C::SPAN_K;
  const int s_beg = z * p.sps;
  const int n = max(0, min(nsp, s_beg + p.sps) - s_beg);               // spans of the slice
  const int tail_span = (K % C::SPAN_K) != 0 ? nsp - 1 : -1;
  const uint32_t row_bytes = uint32_t(K) * 2u;
  const uint32_t x_bytes = uint32_t(M) * row_bytes, ld_bytes = uint32_t(R) * row_bytes;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.x);
  const uint8_t* ldb = reinterpret_cast<const uint8_t*>(p.lora_down);
  uint8_t* xring = smem + wave_u * C::X_RING;
  uint8_t* lring = smem + C::L_OFF;

  // DMA round u: lane l writes slot position (row 4u + l/16, chunk l%16) of
  // its region and reads data chunk (l%16) ^ (row % 16) of that row. x: this
  // wave's rows (past M: row M-1, never stored); lora_down: rank rows 32w ..
  // 32w+31 of the tile (past R: beyond the tensor, read as zeros).
  uint32_t xoff[C::DX], loff[C::DL];
#pragma unroll
  for (int u = 0; u < C::DX; ++u) {
    const int rl = 4 * u + g;
    xoff[u] = uint32_t(min(mw + rl, M - 1)) * row_bytes + uint32_t((r ^ (rl & 15)) << 4);
  }
#pragma unroll
  for (int u = 0; u < C::DL; ++u) {
    const int rank = wave_u * (C::L_ROWS / C::WAVES) + 4 * u + g;
    loff[u] = uint32_t(rank) * row_bytes + uint32_t((r ^ (rank & 15)) << 4);
  }
  // span j of the slice; j >= n: the same loads on an empty descriptor
  auto dma_x = [&](int j) __attribute__((always_inline)) {
    const bool valid = j < n;
    const uint32_t sb = valid ? uint32_t(s_beg + j) * uint32_t(C::ROW_SPAN) : 0u;
    const __amdgpu_buffer_rsrc_t desc = buffer_rsrc(xb + sb, valid ? x_bytes - sb : 0u);
    uint8_t* slot = xring + (j & 1) * C::X_SLOT;
#pragma unroll
    for (int u = 0; u < C::DX; ++u) dma_buf(desc, xoff[u], slot + u * 1024);
  };
  // (R == 0: lora_down may be null and every descriptor is empty)
  auto dma_l = [&](int j) __attribute__((always_inline)) {
    const bool valid = j < n && R > 0;
    const uint32_t sb = valid ? uint32_t(s_beg + j) * uint32_t(C::ROW_SPAN) : 0u;
    const __amdgpu_buffer_rsrc_t desc = buffer_rsrc(ldb + sb, valid ? ld_bytes - sb : 0u);
    uint8_t* slot = lring + (j & 1) * C::L_SLOT + wave_u * (C::L_SLOT / C::WAVES);
#pragma unroll
    for (int u = 0; u < C::DL; ++u) dma_buf(desc, loff[u], slot + u * 1024);
  };

  f32x4_t acc[2][C::RTILES];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int jt = 0; jt < C::RTILES; ++jt) acc[t][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  dma_x(0);
  dma_l(0);
  dma_x(1);

  // outputs: act rows mw + 16t + r from k0 / 2; lanes 0..15 store scale row
  // (block) lane % 8 of the span for row tile lane / 8, 16 consecutive m
  const bool act16 = (K & 31) == 0 && (reinterpret_cast<uintptr_t>(p.act) & 15u) == 0;
  const uintptr_t sc_align = reinterpret_cast<uintptr_t>(p.ascales) | uintptr_t(M);
  const int sc_w = (sc_align & 15u) == 0 ? 16 : (sc_align & 7u) == 0 ? 8 : (sc_align & 3u) == 0 ? 4 : 1;
  const int st_t = (lane >> 3) & 1;
  const int st_row0 = mw + 16 * st_t;
  const int st_nv = max(0, min(16, M - st_row0));
  const uint32_t soff = uint32_t(lane & 7) * uint32_t(M) + uint32_t(min(st_row0, M - 1));
  uint8_t* sc_stage = smem + C::SC_OFF + wave_u * C::SC_BYTES;
  uint32_t code[2][4] = {};
  u32x4 scv = {0u, 0u, 0u, 0u};
  auto store_span = [&](int span) __attribute__((always_inline)) {
    uint8_t* abase = p.act + uint32_t(span) * uint32_t(C::SPAN_K / 2);
    uint8_t* sbase = p.ascales + uint32_t(span) * uint32_t(C::SPAN_K / 16) * uint32_t(M);
    const bool tail = span == tail_span;
    const int k0 = span * C::SPAN_K + 32 * g;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = mw + 16 * t + r;
      if (row < M) {
        uint8_t* dst = abase + uint32_t(row) * uint32_t(K / 2) + uint32_t(16 * g);
        if (act16 && !tail) {
          *reinterpret_cast<u32x4*>(dst) = u32x4{code[t][0], code[t][1], code[t][2], code[t][3]};
        } else {
          if (k0 < K) *reinterpret_cast<u32x2*>(dst) = u32x2{code[t][0], code[t][1]};
          if (k0 + 16 < K) *reinterpret_cast<u32x2*>(dst + 8) = u32x2{code[t][2], code[t][3]};
        }
      }
    }
    if (lane < 16 && st_nv > 0 && span * (C::SPAN_K / 16) + (lane & 7) < K / 16) {
      if (sc_w == 16 && st_nv == 16) {
        *reinterpret_cast<u32x4*>(sbase + soff) = scv;
      } else if (sc_w == 8 && st_nv == 16) {
        *reinterpret_cast<u32x2*>(sbase + soff) = u32x2{scv.x, scv.y};
        *reinterpret_cast<u32x2*>(sbase + soff + 8) = u32x2{scv.z, scv.w};
      } else if (sc_w == 4 && st_nv == 16) {
        uint32_t* d = reinterpret_cast<uint32_t*>(sbase + soff);
        d[0] = scv.x;
        d[1] = scv.y;
        d[2] = scv.z;
        d[3] = scv.w;
      } else {
        const uint64_t lo = uint64_t(scv.x) | (uint64_t(scv.y) << 32), hi = uint64_t(scv.z) | (uint64_t(scv.w) << 32);
#pragma unroll 1
        for (int e = 0; e < st_nv; ++e) sbase[soff + e] = uint8_t((e < 8 ? lo : hi) >> (8 * (e & 7)));
      }
    }
  };

  for (int j = 0; j < n; ++j) {
    const int span = s_beg + j;
    const bool tail = span == tail_span;
    wait_vm_lgkm0<C::VM_J>();                                 // X(j), this wave's part of L(j)
    __builtin_amdgcn_sched_barrier(0);
    if (j > 0) store_span(span - 1);                          // S(j-1)
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();                                             // all of L(j) landed; every wave past span j-1
    __builtin_amdgcn_sched_barrier(0);
    dma_l(j + 1);                                             // L(j+1) into span j-1's slot
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* xs = xring + (j & 1) * C::X_SLOT;
    uint32_t xd[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xs + (16 * t + r) * C::ROW_SPAN + (((4 * g + i) ^ r) << 4));
        xd[t][4 * i] = v.x;
        xd[t][4 * i + 1] = v.y;
        xd[t][4 * i + 2] = v.z;
        xd[t][4 * i + 3] = v.w;
      }
    wait_vm_lgkm0<63>();                                      // the x slot is read
    __builtin_amdgcn_sched_barrier(0);
    dma_x(j + 2);                                             // X(j+2) into it
    __builtin_amdgcn_sched_barrier(0);
    const int k0 = span * C::SPAN_K + 32 * g;
    if (tail) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + 16 * (i >> 3) >= K) xd[t][i] = 0u;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t d[8], sbv;
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = xd[t][8 * b + i];
        quantize_block(d, sbv, code[t][2 * b], code[t][2 * b + 1]);
        sc_stage[(8 * t + 2 * g + b) * 16 + r] = uint8_t(sbv);
      }
    // LoRA-down: B operands of rank tile jt, k-step i from the shared tile,
    // those of k-step i+1 read while k-step i's MFMAs run
    const uint8_t* ls = lring + (j & 1) * C::L_SLOT + r * C::ROW_SPAN;
    auto read_b = [&](int i, u32x4 (&b)[C::RTILES]) __attribute__((always_inline)) {
#pragma unroll
      for (int jt = 0; jt < C::RTILES; ++jt)
        b[jt] = *reinterpret_cast<const u32x4*>(ls + 16 * jt * C::ROW_SPAN + (((4 * g + i) ^ r) << 4));
    };
    auto lora_mfma = [&]<bool TAIL>() __attribute__((always_inline)) {
      u32x4 bb[2][C::RTILES];
      read_b(0, bb[0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i + 1 < 4) read_b(i + 1, bb[(i + 1) & 1]);
        const u32x4 a0 = {xd[0][4 * i], xd[0][4 * i + 1], xd[0][4 * i + 2], xd[0][4 * i + 3]};
        const u32x4 a1 = {xd[1][4 * i], xd[1][4 * i + 1], xd[1][4 * i + 2], xd[1][4 * i + 3]};
#pragma unroll
        for (int jt = 0; jt < C::RTILES; ++jt) {
          u32x4 b = bb[i & 1][jt];
          // k past K: a zero operand (a NaN weight there must not reach valid sums)
          if constexpr (TAIL) b = k0 + 8 * i < K ? b : u32x4{0u, 0u, 0u, 0u};
          acc[0][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                               __builtin_bit_cast(bf16x8, b), acc[0][jt], 0, 0, 0);
          acc[1][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                               __builtin_bit_cast(bf16x8, b), acc[1][jt], 0, 0, 0);
        }
      }
    };
    if (tail) lora_mfma.template operator()<true>();
    else lora_mfma.template operator()<false>();
    wait_vm_lgkm0<63>();
    if (lane < 16) scv = *reinterpret_cast<const u32x4*>(sc_stage + lane * 16);
    wait_vm_lgkm0<63>();                                      // staging read done before the next span's writes
  }
  if (n > 0) store_span(s_beg + n - 1);                       // S(last)

  // lane (col, g) of tile (t, jt) holds rows 16t + 4g .. +3 of this wave's
  // rows, rank 16 jt + col (stored before the drain: the two overlap). A K
  // slice stores plain partial sums, [slice workgroup][ROWS rows][R ranks];
  // producer_reduce_kernel, launched after this kernel, adds them up.
  const bool split = p.ks > 1;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int jt = 0; jt < C::RTILES; ++jt) {
      const int rank = 16 * jt + (lane & 15);
      const int rl = wave * C::ROWS_W + 16 * t + 4 * g;   // first of the lane's four rows in the block
      if (rank < R) {
        if (split) {
          float* dst = p.part + (uint32_t(blockIdx.x) * uint32_t(C::ROWS) + uint32_t(rl)) * uint32_t(R) + uint32_t(rank);
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e * R] = acc[t][jt][e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (m0 + rl + e < M) {
              const __bf16 v = __bf16(acc[t][jt][e]);   // round to nearest even
              p.lora_act_in[uint32_t(m0 + rl + e) * uint32_t(R) + uint32_t(rank)] = __builtin_bit_cast(uint16_t, v);
            }
        }
      }
    }
  wait_vm_lgkm0<0>();                                         // drain the loads past the last span
}

// The wide kernel's split-K reduction: thread u adds VEC consecutive ranks
// of one row over the K slices' partial sums ([row block][slice][ROWS
// rows][R ranks], fp32) in slice order, then rounds them to bf16. Lanes
// take consecutive rank groups, so loads and stores are coalesced; the slice
// loop issues eight slices' loads before it adds them.
constexpr int kReduceThreads = 256;

template <int ROWS, int VEC>
__global__ __launch_bounds__(kReduceThreads) void producer_reduce_kernel(const ProdParams p) {
  const int R = p.R, ks = p.ks;
  const int groups = R / VEC;   // VEC divides R
  const uint32_t u = blockIdx.x * uint32_t(kReduceThreads) + threadIdx.x;
  const uint32_t row_all = u / uint32_t(groups);   // row of the padded row blocks
  const int rb = int(row_all / ROWS), row = int(row_all % ROWS);
  const int r0 = int(u % uint32_t(groups)) * VEC;
  const int m = rb * ROWS + row;
  if (m >= p.M) return;
  const uint32_t slice = uint32_t(ROWS) * uint32_t(R);
  const float* src = p.part + uint32_t(rb) * uint32_t(ks) * slice + uint32_t(row) * uint32_t(R) + uint32_t(r0);
  float s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.f;
#pragma unroll 8
  for (int q = 0; q < ks; ++q) {
    const float* v = static_cast<const float*>(__builtin_assume_aligned(src + uint32_t(q) * slice, 4 * VEC));
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[e] += v[e];
  }
  uint16_t* dst = p.lora_act_in + uint32_t(m) * uint32_t(R) + uint32_t(r0);
  uint16_t b[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) b[e] = __builtin_bit_cast(uint16_t, __bf16(s[e]));   // round to nearest even
  if constexpr (VEC == 4) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{uint32_t(b[0]) | (uint32_t(b[1]) << 16), uint32_t(b[2]) | (uint32_t(b[3]) << 16)};
  } else {
    dst[0] = b[0];
  }
}

// ------------------------------------------------------------------ host side

struct ProdVariant {
  const void* kernel;
  int rtiles, threads, lds;
  int rows;    // rows per workgroup
  bool wide;   // every wave on the same span (producer_wide_kernel)
};

template <int WAVES, int RTILES, int DEPTH>
ProdVariant prod_variant() {
  using C = ProdCfg<WAVES, RTILES, DEPTH>;
  return ProdVariant{reinterpret_cast<const void*>(producer_kernel<C>), RTILES, C::THREADS, C::LDS, C::ROWS, false};
}

template <int RTILES>
ProdVariant prod_wide_variant() {
  using C = WideCfg<RTILES>;
  return ProdVariant{reinterpret_cast<const void*>(producer_wide_kernel<C>), RTILES, C::THREADS, C::LDS, C::ROWS,
                     true};
}

// Instances: narrow kernels for R <= 16 and R <= 32 (8 waves of 16 rows, two
// per SIMD, two ring slots each); the wide kernel (128 rows per workgroup,
// the lora_down tile shared through LDS) with 8, 1 and 2 rank tiles. R = 0
// runs the wide kernel with one rank tile (its lora_down loads read nothing
// and it stores no LoRA sums). Above R = 32 the wide kernel always: a
// narrow kernel for R <= 128 (its operands in two register halves per span)
// was measured slower at every shape tried, 256x3072 to 8192x12288 at R = 64 and 128 (1000x3072
// R=128: 26.2 against 14.4 us; 4096x12288 R=128: 93.3 against 41.3), and
// is not built. At R <= 32 each narrow wave reads its own copy of the
// span's lora_down, 8x the L2 traffic of the wide kernel's shared tile, but
// hides latency with two waves per SIMD; measured:
//  * R <= 32: wide faster from M > 4096 rows or 2^25 elements of x up
//    (16384x3072: 28.5 against 36.2 us; 4096x12288: 28.7 against 33.3;
//    4352x10240: 29.8 against 51.7), narrow faster below (4096x3072: 12.1
//    against 12.5; 1000x3072: 8.1 against 9.2);
//  * R <= 16: narrow faster or equal except where its 16-row blocks
//    overfill the compute units unevenly (4352x10240, 272 blocks: wide 27.6
//    against 36.6 us; 8192x3072, 512 blocks: narrow 15.5 against 18.2).
static const ProdVariant kProdVariants[] = {prod_variant<8, 1, 2>(), prod_variant<8, 2, 2>(),
                                            prod_wide_variant<8>(), prod_wide_variant<1>(),
                                            prod_wide_variant<2>()};

static int prod_variant_index(int M, int K, int R, int cus) {
  if (R > 32) return 2;
  if (R == 0) return 3;
  const int rbs = (M + 15) / 16;                        // narrow row blocks
  const int full = rbs / cus, part = rbs % cus;         // whole rounds, the last round's blocks
  const bool uneven = full >= 1 && part > 0 && part * 4 <= cus * 3;   // last round <= 3/4 full
  if (R <= 16) return uneven ? 3 : 0;
  return rbs > cus || size_t(M) * size_t(K) >= (size_t(1) << 25) ? 4 : 1;
}

static std::atomic<int> g_cus[64];

static int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 256;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Scratch of the split-K reduction: a fixed region of arrival counters (one
// per row block of a narrow kernel; the same bytes in every call, so they
// stay zero between calls), then the partial sums, at most kProdMaxPartBytes
// (K is split fewer ways where more would be needed; both entry points plan
// alike). The wide kernel's reduction is a second launch and uses no counter.
constexpr int kProdMaxCounters = 1024;
constexpr size_t kProdCountBytes = kProdMaxCounters * 4;
constexpr size_t kProdMaxPartBytes = size_t(QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES) - kProdCountBytes;
static_assert(QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES > int(kProdCountBytes), "counters fit the fixed scratch");

struct ProdLaunch {
  int ks, sps;
  size_t part_bytes;   // partial sums after the counters; 0: no scratch
};

// K slices, so that the workgroups of all row blocks spread over the compute
// units in one round. Narrow kernel: one slice when the row blocks alone
// fill every compute unit or its waves would have a single span each; else
// up to one workgroup per compute unit, down to one span per wave (measured
// against splitting only from 4 spans per wave, 2 kept, with the workgroup
// slots of two per CU: 1000x3072 R=16 6.8 against 8.2 us, 2048x3072 R=32
// 9.3 against 11.1, 3000x12288 R=32 32.4 against 37.3; filling both slots
// per CU was slower from 1500 rows on). Wide kernel (its waves share every
// span, and its LDS fills a compute unit): likewise, down to one span per
// slice (256x3072 R=64 9.5 us against 16.3 at four spans per slice,
// 1000x12288 R=128 19.9 against 38.7 with at most 8 slices);
// producer_reduce_kernel then adds the slices. Both: no slice left empty,
// and partial sums within kProdMaxPartBytes.
static ProdLaunch prod_plan(int vi, int M, int K, int R) {
  const ProdVariant& v = kProdVariants[vi];
  const int rbs = (M + v.rows - 1) / v.rows, nsp = (K + 127) / 128;
  const int waves = v.threads / kWave;
  const int cus = compute_units();
  ProdLaunch pl{1, nsp, 0};
  int ks = 1;
  if (rbs < cus && rbs <= kProdMaxCounters) {
    if (v.wide) {
      ks = min(nsp, max(1, cus / rbs));
    } else if (nsp >= 2 * waves) {
      ks = min(nsp / waves, max(1, cus / rbs));
    }
    if (R > 0) {
      const size_t per_slice = size_t(rbs) * size_t(v.rows) * size_t(R) * 4;
      const int cap = v.wide ? kProdMaxWideSlices : kProdMaxSlices;
      ks = int(min(size_t(min(ks, cap)), max(size_t(1), kProdMaxPartBytes / per_slice)));
    }
  }
  if (ks > 1) {
    const int sps = (nsp + ks - 1) / ks;
    pl.ks = (nsp + sps - 1) / sps;
    pl.sps = sps;
  }
  if (pl.ks > 1 && R > 0) pl.part_bytes = size_t(rbs) * size_t(pl.ks) * size_t(v.rows) * size_t(R) * 4;
  return pl;
}

// Scratch of the split-K reduction, one per (device, stream): calls on one
// stream run in order, so each call finds the counters it needs at zero
// (every call returns them there) and no other call's partial sums in its
// way; calls on different streams never share one. Grown on demand, zeroed
// when allocated, kept until the process ends.
struct ProdScratch {
  void* ptr = nullptr;
  size_t bytes = 0;
};
static std::map<std::pair<int, void*>, ProdScratch> g_prod_scratch;
static std::mutex g_prod_scratch_mu;

static int prod_scratch(size_t need, void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_W4A4_EDEVICE;
  std::lock_guard<std::mutex> lock(g_prod_scratch_mu);
  ProdScratch& s = g_prod_scratch[{dev, stream}];
  if (s.bytes < need) {
    if (s.ptr && hipFree(s.ptr) != hipSuccess) return GEMM_W4A4_ENOMEM;   // waits for the device
    s.ptr = nullptr;
    s.bytes = 0;
    void* ptr = nullptr;
    if (hipMalloc(&ptr, need) != hipSuccess) return GEMM_W4A4_ENOMEM;
    if (hipMemset(ptr, 0, need) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      (void)hipFree(ptr);
      return GEMM_W4A4_ENOMEM;
    }
    s.ptr = ptr;
    s.bytes = need;
  }
  *out = s.ptr;
  return GEMM_W4A4_OK;
}

}  // namespace w4a4

// Scratch of quantize_w4a4_act_noalloc: one copy per GPU, held until the
// process ends. The arrival counters at its start are zero when the module
// is loaded and every call returns them to zero. Host code must not pass
// `scratch` itself to a kernel (it names a host-side stand-in): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES];

namespace w4a4 {

static std::atomic<uintptr_t> g_noalloc_scratch[64];
static std::mutex g_noalloc_mu;

static int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_W4A4_EDEVICE;
  uintptr_t ptr = g_noalloc_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    ptr = g_noalloc_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      void* sym = nullptr;   // this device's copy of the array (the device is current)
      if (hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)) != hipSuccess || !sym) return GEMM_W4A4_EDEVICE;
      ptr = reinterpret_cast<uintptr_t>(sym);
      g_noalloc_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = reinterpret_cast<void*>(ptr);
  return GEMM_W4A4_OK;
}

static bool prod_sizes_ok(int M, int K, int R) {
  if (!(M >= 1 && K >= 16 && K % 16 == 0 && R >= 0 && R <= QUANTIZE_W4A4_MAX_R)) return false;
  const int64_t lim = int64_t(1) << 31;
  return int64_t(M) * K * 2 < lim && int64_t(R) * K * 2 < lim && int64_t(M) * R * 2 < lim;
}

// Checks, plan, scratch and launch shared by both entry points; `noalloc`
// takes the scratch from the fixed array instead of the library's buffer.
static int quantize_run(const uint16_t* x, const uint16_t* lora_down, uint8_t* act, uint8_t* ascales,
                        uint16_t* lora_act_in, int M, int K, int R, void* stream, bool noalloc) {
  if (!prod_sizes_ok(M, K, R)) return GEMM_W4A4_EINVAL;
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
  const int vi = prod_variant_index(M, K, R, compute_units());
  const ProdVariant& v = kProdVariants[vi];
  const ProdLaunch pl = prod_plan(vi, M, K, R);
  void* buf = nullptr;
  if (pl.part_bytes > 0) {
    const size_t need = kProdCountBytes + pl.part_bytes;
    int rc;
    if (noalloc) {
      if (need > size_t(QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES)) return GEMM_W4A4_ESCRATCH;
      rc = noalloc_scratch(&buf);
    } else {
      rc = prod_scratch(need, stream, &buf);
    }
    if (rc != GEMM_W4A4_OK) return rc;
  }
  uint8_t* sb = static_cast<uint8_t*>(buf);
  ProdParams prm{x, lora_down, act, ascales, lora_act_in, M, K, R, pl.ks, pl.sps,
                 sb ? reinterpret_cast<float*>(sb + kProdCountBytes) : nullptr, reinterpret_cast<uint32_t*>(sb)};
  void* args[] = {&prm};
  const int rbs = (M + v.rows - 1) / v.rows;
  hipError_t e = hipLaunchKernel(v.kernel, dim3(rbs * pl.ks), dim3(v.threads), args, 0, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && v.wide && pl.part_bytes > 0) {
    // four ranks per thread (8-byte stores) where R and lora_act_in allow
    const bool vec4 = R % 4 == 0 && (reinterpret_cast<uintptr_t>(lora_act_in) & 7u) == 0;
    const size_t units = size_t(rbs) * size_t(v.rows) * size_t(vec4 ? R / 4 : R);
    const void* rk = vec4 ? reinterpret_cast<const void*>(producer_reduce_kernel<WideCfg<8>::ROWS, 4>)
                          : reinterpret_cast<const void*>(producer_reduce_kernel<WideCfg<8>::ROWS, 1>);
    e = hipLaunchKernel(rk, dim3(unsigned((units + kReduceThreads - 1) / kReduceThreads)), dim3(kReduceThreads), args,
                        0, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? GEMM_W4A4_OK : GEMM_W4A4_ELAUNCH;
}

static int quantize_plan(int M, int K, int R, quantize_w4a4_plan_t* out) {
  if (!out || !prod_sizes_ok(M, K, R)) return GEMM_W4A4_EINVAL;
  const int vi = prod_variant_index(M, K, R, compute_units());
  const ProdVariant& v = kProdVariants[vi];
  const ProdLaunch pl = prod_plan(vi, M, K, R);
  const int rbs = (M + v.rows - 1) / v.rows;
  quantize_w4a4_plan_t q{};
  q.variant = vi;
  q.wide = v.wide ? 1 : 0;
  q.rank_tiles = v.rtiles;
  q.rows = v.rows;
  q.threads = v.threads;
  q.lds_bytes = v.lds;
  q.row_blocks = rbs;
  q.k_slices = pl.ks;
  q.spans_per_slice = pl.sps;
  q.grid = rbs * pl.ks;
  q.launches = v.wide && pl.part_bytes > 0 ? 2 : 1;
  q.scratch_bytes = pl.part_bytes > 0 ? (long long)(kProdCountBytes + pl.part_bytes) : 0;
  *out = q;
  return GEMM_W4A4_OK;
}

}  // namespace w4a4

extern "C" int quantize_w4a4_act_plan(int M, int K, int R, quantize_w4a4_plan_t* plan) {
  return w4a4::quantize_plan(M, K, R, plan);
}

extern "C" int quantize_w4a4_act(const uint16_t* x, const uint16_t* lora_down, uint8_t* act,
                                 uint8_t* ascales, uint16_t* lora_act_in, int M, int K, int R,
                                 void* stream) {
  return w4a4::quantize_run(x, lora_down, act, ascales, lora_act_in, M, K, R, stream, false);
}

extern "C" int quantize_w4a4_act_noalloc(const uint16_t* x, const uint16_t* lora_down, uint8_t* act,
                                         uint8_t* ascales, uint16_t* lora_act_in, int M, int K, int R,
                                         void* stream) {
  return w4a4::quantize_run(x, lora_down, act, ascales, lora_act_in, M, K, R, stream, true);
}
