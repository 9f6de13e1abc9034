// gemm_mxfp4.hip — the fused operator with MXFP4 operands, on gfx950's scaled FP4 MFMA.
//
// y[m,n] = wcscale[n] * sum_k A[m,k] W[n,k] + bias[n] + sum_r la[m,r] lu[r,n]
//
// A and W are E2M1 codes (two per byte, low nibble = even k) times one UE8M0
// scale 2^(b-127) per 32 consecutive k. The DeepGEMM FP4 indexer page ("Step
// 0") describes this pairing: E2M1 data whose UE8M0 block scale the matrix
// unit applies itself, the dequantized value never existing in a register;
// the 32-wide block is the OCP MX one gfx950's instruction takes. The affine
// and the LoRA residual are the SVDQuant W4A4 on Blackwell page's (sections 2,
// 6.3, 6.6), shared with the NVFP4 kernel (w4a4_epilogue.hpp).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 A and B (cbsz = blgp = 4) computes
// a 32x32 tile over 64 values of k and applies the scales itself. Lane l holds
// row (A) or column (B) l % 32 and k = 32*(l/32) .. +31 as the 32 nibbles of
// 16 bytes, and supplies the scale of exactly that 32-block as one byte of a
// VGPR chosen by op_sel (measured on gfx950 with a one-wave probe against a
// host reference, every op_sel). So nothing is decoded: operand bytes and
// scale bytes go HBM -> LDS by direct-to-LDS DMA and LDS -> MFMA unchanged,
// and the kernel is a DMA ring feeding MFMAs.
//
// Pipeline (LDS ring of S stages, one stage = 128 k = two MFMA k-steps,
// prefetch distance PF = S - 1): iteration st runs k-step 0 of stage st while
// it DMAs stage st+PF and reads k-step 1's operands, waits for its own DMA of
// stage st+1 and meets the workgroup barrier, then runs k-step 1 while it
// reads stage st+1's k-step 0 operands and scales. Every read of stage st-1
// happened before the previous barrier, so DMA(st+PF) may refill buffer
// (st-1) % S from the start of iteration st.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "gemm_w4a4.h"
#include "w4a4_common.hpp"
#include "w4a4_epilogue.hpp"
#include "w4a4_host.hpp"
#include "w4a4_layout.hpp"

namespace w4a4 {

// D += (A * 2^(sa_byte - 127)) (B * 2^(sb_byte - 127)) over 64 k, FP4 operands;
// byte SEL of sa / sb is the scale (one per lane, for its 32 k).
template <int SEL>
__device__ __forceinline__ f32x16 mfma_fp4(u32x4 a, u32x4 b, f32x16 c, uint32_t sa, uint32_t sb) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  const v8i av = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};   // FP4 uses the low 4 dwords
  const v8i bv = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, SEL, int(sa), SEL, int(sb));
}

// The act-scale windows of the AWIN flavour (k-block rows of BM + 4 bytes)
// fit in the stage's scale DMA rounds.
template <class C>
constexpr bool kAwinRoom = C::KBLK * (C::BM + 4 + C::BN) <= C::SCALE_ROUNDS * C::THREADS * 4;

// GENERAL = false (fast): K % 128 == 0, M % 4 == 0, N % 8 == 0, 4-byte aligned scales and
// the LoRA conditions of the shared epilogue's fast path (R % 8 == 0, 16-byte
// aligned LoRA operands); scales move by DMA into LDS. GENERAL = true: any
// valid shape; each lane loads its own scale bytes one stage ahead.
// F16: LoRA operands and output in binary16 (else bfloat16).
// AWIN (fast flavour, any M): each k-block row of act scales moves as a window
// of BM + 4 bytes from the 4-byte boundary at or below its first byte, so
// that its 4-byte DMA pieces stay aligned when M % 4 != 0; the reader adds the
// row's offset into its window (see act_window).
// PART (fast flavour without windows, K % 128 == 0): workgroup (tile,
// blockIdx.y) runs slice blockIdx.y of gridDim.y of the tile's K stages and
// stores float32 sums (see epilogue); split_k_reduce adds the slices.
template <class C, bool GENERAL, bool F16, bool AWIN = false, bool PART = false>
__global__ __launch_bounds__(C::THREADS, C::OCC * C::THREADS / 256) void gemm_mxfp4_kernel(
    const Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  constexpr int P_ROUNDS = C::PACKED_BYTES / (C::THREADS * 16);   // packed DMA rounds per stage
  constexpr int A_ROUNDS = C::B_OFF / (C::THREADS * 16);
  constexpr int S_ROUNDS = GENERAL ? 0 : C::SCALE_ROUNDS;        // scale DMA rounds per stage
  constexpr int DMA_N = P_ROUNDS + S_ROUNDS;                     // DMA per thread per stage
  constexpr int T = C::MI + C::NI;                               // operand tiles per wave
  constexpr int G = C::MI * C::NI;                               // MFMAs per k-step
  constexpr int ROWS_PER_ROUND = C::THREADS * 16 / C::ROW_BYTES;
  constexpr int PF = C::STAGES - 1;                              // prefetch distance in stages
  static_assert((PF - 1) * DMA_N < 64, "vmcnt range");
  static_assert(ROWS_PER_ROUND % 32 == 0, "the chunk swizzle repeats every 32 rows");
  // each MFMA group issues at most one operand read, tile q - (G - T) (k-step
  // 0) or q (k-step 1): every tile needs a group (a 32x96 wave tile, 4 tiles
  // for 3 MFMAs, would leave one unread)
  static_assert(T <= G, "one operand tile read per MFMA group");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave / C::WN, wn = wave % C::WN;

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = (p.tm0 + tm) * C::BM, n0 = tn * C::BN;
  const int M = p.M, N = p.N;
  const int rowbytes = p.K >> 1;             // packed row stride
  // the stages [ks0, ks1) this workgroup runs: all, or its K slice; the
  // operand pointers start at the first of them
  static_assert(!PART || (!GENERAL && !AWIN), "K slices run on the fast flavour");
  const int nst_all = (p.K + C::BK - 1) / C::BK;
  const int ks0 = PART ? int(blockIdx.y) * nst_all / int(gridDim.y) : 0;
  const int ks1 = PART ? (int(blockIdx.y) + 1) * nst_all / int(gridDim.y) : nst_all;
  const uint8_t* const act = p.act + (PART ? size_t(ks0) * C::ROW_BYTES : 0);
  const uint8_t* const wgt = p.wgt + (PART ? size_t(ks0) * C::ROW_BYTES : 0);
  const uint8_t* const ascales = p.ascales + (PART ? size_t(ks0) * C::KBLK * size_t(M) : 0);
  const uint8_t* const wscales = p.wscales + (PART ? size_t(ks0) * C::KBLK * size_t(N) : 0);
  const int K = PART ? (ks1 - ks0) * C::BK : p.K;   // k of this workgroup
  const int kbytes = K >> 1;                 // packed bytes of a row it reads
  const int KB = K >> 5;                     // scale blocks along k
  const int nst = (K + C::BK - 1) / C::BK;
  const int last = nst - 1;

  // ---- packed DMA (as the NVFP4 kernel's, 16-byte pieces only: K % 32 == 0
  // makes rows a multiple of 16 bytes). Slot q = u*THREADS + tid of a stage's
  // packed region holds the bytes of data chunk cp ^ swz(row) of its row.
  const int dma_row0 = tid * 16 / C::ROW_BYTES;
  const uint32_t dma_inrow = uint32_t(((tid & 3) ^ swz(dma_row0)) * 16);
  const int full_stages = kbytes / C::ROW_BYTES;
  auto dma_packed = [&](int st, int buf, int u) __attribute__((always_inline)) {
    uint8_t* stage = smem + (buf % C::STAGES) * C::STAGE_BYTES;
    const bool is_b = u >= A_ROUNDS;
    const int ur = is_b ? u - A_ROUNDS : u;
    const uint32_t k0 = uint32_t(st * C::ROW_BYTES);
    // pieces past the row end (partial last stage only) re-read the row start;
    // their 32-blocks are masked to zero where the operands are used
    const uint32_t kin = (st >= full_stages && dma_inrow + k0 + 16 > uint32_t(kbytes)) ? 0u : k0 + dma_inrow;
    const int row = min((is_b ? n0 : m0) + dma_row0 + ur * ROWS_PER_ROUND, (is_b ? N : M) - 1);
    const uint8_t* src = (is_b ? wgt : act) + (uint32_t(row) * uint32_t(rowbytes) + kin);
    dma<16>(src, stage + (u * C::THREADS + wave_u * 64) * 16);
  };
  // ---- act-scale windows (AWIN). Row stride of the act scales in LDS: BM,
  // or BM + 4 with windows; the wgt scales follow the act ones.
  constexpr int SW = AWIN ? C::BM + 4 : C::BM;
  constexpr int SB_OFF = C::SA_OFF + C::KBLK * SW;
  static_assert(!AWIN || kAwinRoom<C>, "act-scale windows need room in the stage's scale area");
  // Start of k-block kb's window: the 4-byte boundary at or below its first
  // byte (kb*M + m0), clamped so that the window ends inside the tensor (the
  // host requires KB*M >= SW; KB*M % 4 == 0 as K % 128 == 0). The tile's
  // valid rows then always lie inside the window.
  auto act_window = [&](int kb) __attribute__((always_inline)) {
    const uint32_t first = uint32_t(kb) * uint32_t(M) + uint32_t(m0);
    return min(first & ~3u, uint32_t(KB) * uint32_t(M) - uint32_t(SW));
  };
  // Offset of the tile's row 0 in the window of k-block kb (clamped as the DMA).
  auto act_shift = [&](int kb) __attribute__((always_inline)) {
    const int k = min(kb, KB - 1);
    return int(uint32_t(k) * uint32_t(M) + uint32_t(m0) - act_window(k));
  };
  // ---- scale DMA (fast flavour): 4-byte pieces = 4 consecutive rows of one
  // k-block, the global [K/32][rows] order kept: [4][BM] act then [4][BN]
  // wgt. Blocks past K read the last block (their data is masked); rows past
  // the edge read the last 4 rows (only discarded outputs); padding lanes
  // re-read a valid piece.
  auto dma_scales = [&](int st, int buf, int v) __attribute__((always_inline)) {
    uint8_t* stage = smem + (buf % C::STAGES) * C::STAGE_BYTES;
    const int o = (v * C::THREADS + tid) * 4;
    const uint8_t* src;
    if (o < C::KBLK * SW) {
      const int kb = min(st * C::KBLK + o / SW, KB - 1);
      if constexpr (AWIN)
        src = ascales + act_window(kb) + uint32_t(o % SW);
      else
        src = ascales + uint32_t(kb) * uint32_t(M) + uint32_t(min(m0 + o % C::BM, M - 4));
    } else {
      const int ob = min(o - C::KBLK * SW, C::KBLK * C::BN - 4);
      const int kb = min(st * C::KBLK + ob / C::BN, KB - 1);
      src = wscales + uint32_t(kb) * uint32_t(N) + uint32_t(min(n0 + ob % C::BN, N - 4));
    }
    dma<4>(src, stage + C::SA_OFF + (v * C::THREADS + wave_u * 64) * 4);
  };
  auto dma_round = [&](int st, int buf, int u) __attribute__((always_inline)) {
    if (u < P_ROUNDS)
      dma_packed(st, buf, u);
    else
      dma_scales(st, buf, u - P_ROUNDS);
  };

  // ---- operand reads. Lane (l32, g) of tile t reads row r = (wave's first
  // row) + 32t' + l32 of the stage, data chunk 2s + g for k-step s (k =
  // 32(2s+g) .. +31 of the stage, scale block 2s + g). Tiles 0 .. MI-1 are
  // act rows (the MFMA's B operand), MI .. T-1 wgt rows (its A operand).
  const int ra = wm * C::TM + l32, rb = wn * C::TN + l32;
  auto read_tile = [&](int st, int s, int t) __attribute__((always_inline)) {
    const uint8_t* stage = smem + (st % C::STAGES) * C::STAGE_BYTES;
    const int r = t < C::MI ? ra + 32 * t : rb + 32 * (t - C::MI);
    const int off = t < C::MI ? C::A_OFF : C::B_OFF;
    return *reinterpret_cast<const u32x4*>(stage + off + r * C::ROW_BYTES + (((2 * s + g) ^ swz(r)) << 4));
  };
  // The fast flavour's two scale bytes of a stage for tile t (blocks g and
  // 2+g), read into two registers; combined (scales_join) only where they are
  // next used, so that no LDS read is waited for in the slot that issues it.
  auto read_scale_bytes = [&](int st, int t, uint32_t& b0, uint32_t& b1) __attribute__((always_inline)) {
    const uint8_t* stage = smem + (st % C::STAGES) * C::STAGE_BYTES;
    if (AWIN && t < C::MI) {
      const uint8_t* q = stage + C::SA_OFF + ra + 32 * t;
      b0 = q[g * SW + act_shift(st * C::KBLK + g)];
      b1 = q[(2 + g) * SW + act_shift(st * C::KBLK + 2 + g)];
      return;
    }
    const uint8_t* q = t < C::MI ? stage + C::SA_OFF + ra + 32 * t
                                 : stage + SB_OFF + rb + 32 * (t - C::MI);
    const int rows = t < C::MI ? C::BM : C::BN;
    b0 = q[g * rows];
    b1 = q[(2 + g) * rows];
  };
  // The lane's two scale bytes of a stage (blocks g and 2+g) as bytes 0 and 1.
  auto read_scales = [&](int st, int t) __attribute__((always_inline)) {
    if constexpr (!GENERAL) {
      uint32_t b0, b1;
      read_scale_bytes(st, t, b0, b1);
      return b0 | (b1 << 8);
    } else {
      const bool is_a = t < C::MI;
      const uint8_t* src = is_a ? ascales : wscales;
      const int nrows = is_a ? M : N;
      const int row = min((is_a ? m0 + ra + 32 * t : n0 + rb + 32 * (t - C::MI)), nrows - 1);
      const int kb0 = min(st * C::KBLK + g, KB - 1), kb1 = min(st * C::KBLK + 2 + g, KB - 1);
      return uint32_t(src[uint32_t(kb0) * uint32_t(nrows) + uint32_t(row)]) |
             (uint32_t(src[uint32_t(kb1) * uint32_t(nrows) + uint32_t(row)]) << 8);
    }
  };

  f32x16 acc[C::NI][C::MI];
#pragma unroll
  for (int j = 0; j < C::NI; ++j)
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // One k-step: MFMA group q (tile pair j, i) followed by `op(q)`, fenced.
  // 32-blocks past K (k-step s of stage st, lane half g) get zero act bytes.
  auto kstep = [&]<int S>(int st, const u32x4 (&o)[T], const uint32_t (&sc)[T], auto op)
      __attribute__((always_inline)) {
    const bool live = GENERAL ? st * C::KBLK + 2 * S + g < KB : true;   // fast: K % 128 == 0
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int j = q / C::MI, i = q % C::MI;
      const u32x4 a = (GENERAL && !live) ? u32x4{0u, 0u, 0u, 0u} : o[i];
      acc[j][i] = mfma_fp4<S>(o[C::MI + j], a, acc[j][i], sc[C::MI + j], sc[i]);
      op(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: the epilogue's side DMA, then DMA stages 0 .. PF-1, wait
  // for stage 0, publish it, read its k-step 0 operands and its scales.
  EpiRegs epi_regs;
  epilogue_prefetch<C, GENERAL>(p, smem, tid, m0, n0, epi_regs);
  u32x4 O0[T], O1[T];
  uint32_t SC[T], SCn[T], SCh[T];   // SCh: the fast flavour's second scale bytes
#pragma unroll
  for (int s = 0; s < PF; ++s)
#pragma unroll
    for (int u = 0; u < DMA_N; ++u) dma_round(min(s, last), s, u);
  wait_vm_lgkm0<(PF - 1) * DMA_N>();
  wg_barrier();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    O0[t] = read_tile(0, 0, t);
    SC[t] = read_scales(0, t);
  }

  for (int st = 0; st < nst; ++st) {
    // k-step 0 of stage st; alongside: DMA(st+PF) and k-step 1's operands
    kstep.template operator()<0>(st, O0, SC, [&](int q) __attribute__((always_inline)) {
#pragma unroll
      for (int u = q; u < DMA_N; u += G) dma_round(min(st + PF, last), st + PF, u);
      const int t = q - (G - T);
      if (t >= 0 && t < T) O1[t] = read_tile(st, 1, t);
    });
    // stage st+1 complete in this wave's view (the ops after it are DMA(st+2)
    // .. DMA(st+PF), plus, in the general flavour, scale loads, which only
    // makes the wait longer); publish it
    wait_vm_lgkm0<(PF - 1) * DMA_N>();
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 1 of stage st; alongside: stage st+1's k-step 0 operands and
    // scales (fast flavour: the scale bytes first, combined after the k-step)
    kstep.template operator()<1>(st, O1, SC, [&](int q) __attribute__((always_inline)) {
      if constexpr (GENERAL) {
        if (q < T) O0[q] = read_tile(st + 1, 0, q);
        const int t = q - (G - T);
        if (t >= 0 && t < T) SCn[t] = read_scales(st + 1, t);
      } else {
        if (q < T) read_scale_bytes(st + 1, q, SCn[q], SCh[q]);
        const int t = q - (G - T);
        if (t >= 0 && t < T) O0[t] = read_tile(st + 1, 0, t);
      }
    });
#pragma unroll
    for (int t = 0; t < T; ++t) SC[t] = GENERAL ? SCn[t] : (SCn[t] | (SCh[t] << 8));
  }
  wait_vm_lgkm0<0>();   // drain the prefetches past the last stage

  epilogue<C, GENERAL, F16, PART>(acc, p, smem, tid, m0, n0, epi_regs);
}

// ------------------------------------------------------------------ host side

// Rounds of the chip x the work of one round, as for NVFP4; nothing is
// decoded, so the per-tile factor is the LDS operand traffic per MFMA, which
// grows as (TM + TN) / (TM * TN) for a wave tile TM x TN.
template <class C>
VariantDesc mx_variant() {
  static const void* const k[2][3] = {
      {reinterpret_cast<const void*>(gemm_mxfp4_kernel<C, true, false>),
       reinterpret_cast<const void*>(gemm_mxfp4_kernel<C, false, false>),
       reinterpret_cast<const void*>(gemm_mxfp4_kernel<C, false, false, kAwinRoom<C>>)},
      {reinterpret_cast<const void*>(gemm_mxfp4_kernel<C, true, true>),
       reinterpret_cast<const void*>(gemm_mxfp4_kernel<C, false, true>),
       reinterpret_cast<const void*>(gemm_mxfp4_kernel<C, false, true, kAwinRoom<C>>)}};
  constexpr double tm = double(C::TM), tn = double(C::TN);
  constexpr double per_elem = 1.0 + 16.0 * (tm + tn) / (tm * tn);
  constexpr double ref = 1.0 + 16.0 * (128.0 + 96.0) / (128.0 * 96.0);   // the 128x96 wave tile
  return describe<C>(k, kAwinRoom<C>, per_elem / ref);
}

static const VariantDesc kMxVariants[] = {mx_variant<MxCfg256x192>(), mx_variant<MxCfg128x128>()};
static constexpr int kNumMxVariants = int(sizeof(kMxVariants) / sizeof(kMxVariants[0]));
// What a launch costs besides its k-loop, in k-stages of a full round of
// 256x192 tiles: a 4096x3072 launch over one stage (K = 128) takes about
// 10.6 us against 0.78 us per added stage.
static constexpr double kMxLaunchStages = 12.7;
// The instance compiled with K-sliced workgroups (128x128), as the tail of a
// split plan, its kernels [F16] and the reduction.
static constexpr int kMxPartVariant = 1;
static const void* const kMxPartKernel[2] = {
    reinterpret_cast<const void*>(gemm_mxfp4_kernel<MxCfg128x128, false, false, false, true>),
    reinterpret_cast<const void*>(gemm_mxfp4_kernel<MxCfg128x128, false, true, false, true>)};
static const void* const kMxReduceKernel[2] = {reinterpret_cast<const void*>(split_k_reduce<false>),
                                               reinterpret_cast<const void*>(split_k_reduce<true>)};
// K slices need whole stages, N % 8 == 0 and the fast flavour without act-scale
// windows on the 128-row tail (M % 4 == 0).
static bool mx_slices_ok(int M, int N, int K, int R) {
  return K % 128 == 0 && N % 8 == 0 && M % 4 == 0 && (R == 0 || R % 8 == 0);
}

// K a multiple of the 32-wide scale block; every tensor below 2^31 bytes.
static bool mx_sizes_ok(int M, int N, int K, int R) {
  if (!(M >= 1 && N >= 1 && K >= 32 && K % 32 == 0 && R >= 0 && R <= GEMM_W4A4_MAX_R)) return false;
  const int64_t lim = int64_t(1) << 31;
  const int64_t m = M, n = N, k = K, r = R;
  return m * k / 2 < lim && n * k / 2 < lim && m * n * 2 < lim && m * r * 2 < lim && r * n * 2 < lim;
}

// Fast flavour: K % 128 == 0, N % 8 == 0, 4-byte aligned scales, LoRA as for
// NVFP4; M % 4 != 0 takes the act-scale windows where the tile has room for
// them and the tensor holds at least one window (K/32 * M >= BM + 4).
static int mx_flavour(const VariantDesc& v, int M, int N, int K, int R, uintptr_t scales, uintptr_t lora) {
  const bool fast = K % 128 == 0 && N % 8 == 0 && (scales & 3u) == 0 &&
                    (R == 0 || (R % 8 == 0 && (lora & 15u) == 0));
  const bool awin = v.has_window && int64_t(K / 32) * M >= v.block_m + 4;
  return !fast ? 0 : M % 4 == 0 ? 1 : awin ? 2 : 0;
}

int mx_plan(int variant, int M, int N, int K, int R, gemm_w4a4_plan_t* pl) {
  if (!pl || !mx_sizes_ok(M, N, K, R) || variant < -1 || variant >= kNumMxVariants) return GEMM_W4A4_EINVAL;
  const Choice c = variant >= 0 ? Choice{variant, -1, M, 1}
                                 : choose_plan(kMxVariants, kNumMxVariants, M, N, K, kMxLaunchStages,
                                               mx_slices_ok(M, N, K, R) ? kMxPartVariant : -1);
  const int rc = plan_choice(kMxVariants, c, M, N, K, R, pl);
  if (rc == GEMM_W4A4_OK) fill_registers(kMxVariants[c.main], mx_flavour(kMxVariants[c.main], M, N, K, R, 0, 0), pl);
  return rc;
}

int mx_run(int variant, bool f16, const CallArgs& a) {
  if (!mx_sizes_ok(a.M, a.N, a.K, a.R) || variant < -1 || variant >= kNumMxVariants) return GEMM_W4A4_EINVAL;
  int rc = check_call(a, 32);
  if (rc != GEMM_W4A4_OK) return rc;
  gemm_w4a4_plan_t pl;
  if (mx_plan(variant, a.M, a.N, a.K, a.R, &pl) != GEMM_W4A4_OK) return GEMM_W4A4_EINVAL;
  rc = check_device();
  if (rc != GEMM_W4A4_OK) return rc;
  const uintptr_t scales = uintptr_t(a.ascales) | uintptr_t(a.wscales);
  const uintptr_t lora = a.R > 0 ? (uintptr_t(a.lora_act_in) | uintptr_t(a.lora_up)) : 0u;
  return launch_plan(kMxVariants, pl, a, [&](const VariantDesc& v) {
    return v.kernel[f16 ? 1 : 0][mx_flavour(v, a.M, a.N, a.K, a.R, scales, lora)];
  }, [&](int rows, int splits, int row0) -> int {
    // the fast flavour without windows on the tail instance, and 16-byte
    // aligned float32 sums in the output
    const VariantDesc& t = kMxVariants[kMxPartVariant];
    if (mx_flavour(t, a.M, a.N, a.K, a.R, scales, lora) != 1 || (uintptr_t(a.out) & 15u) != 0)
      return GEMM_W4A4_EINVAL;
    return launch_slices(kMxPartKernel[f16 ? 1 : 0], kMxReduceKernel[f16 ? 1 : 0], t, rows, splits, row0, a);
  });
}

// The NVFP4 family's plan and launch (gemm_w4a4.hip), for the format-generic calls.
int nv_plan(int variant, int M, int N, int K, int R, gemm_w4a4_plan_t* pl);
int nv_run(int variant, bool f16, const CallArgs& a);

}  // namespace w4a4

using namespace w4a4;

extern "C" int gemm_mxfp4(const uint8_t* act, const uint8_t* ascales, const uint8_t* wgt,
                          const uint8_t* wscales, const float* wcscale, const float* bias,
                          const uint16_t* lora_act_in, const uint16_t* lora_up, uint16_t* out,
                          int M, int N, int K, int R, void* stream) {
  return mx_run(-1, false, CallArgs{act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                                    M, N, K, R, stream});
}

extern "C" int gemm_mxfp4_f16(const uint8_t* act, const uint8_t* ascales, const uint8_t* wgt,
                              const uint8_t* wscales, const float* wcscale, const float* bias,
                              const uint16_t* lora_act_in, const uint16_t* lora_up, uint16_t* out,
                              int M, int N, int K, int R, void* stream) {
  return mx_run(-1, true, CallArgs{act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                                   M, N, K, R, stream});
}

extern "C" int gemm_mxfp4_plan(int M, int N, int K, int R, gemm_w4a4_plan_t* plan) {
  return mx_plan(-1, M, N, K, R, plan);
}

extern "C" int gemm_mxfp4_num_variants(void) { return kNumMxVariants; }

extern "C" int gemm_mxfp4_variant_info(int variant, gemm_w4a4_plan_t* plan) {
  if (!plan || variant < 0 || variant >= kNumMxVariants) return GEMM_W4A4_EINVAL;
  fill_static(kMxVariants[variant], variant, plan);
  return GEMM_W4A4_OK;
}

extern "C" int gemm_w4a4_run(int format, int out_f16, int variant, const uint8_t* act,
                             const uint8_t* ascales, const uint8_t* wgt, const uint8_t* wscales,
                             const float* wcscale, const float* bias, const uint16_t* lora_act_in,
                             const uint16_t* lora_up, uint16_t* out, int M, int N, int K, int R,
                             void* stream) {
  if (out_f16 != 0 && out_f16 != 1) return GEMM_W4A4_EINVAL;
  const CallArgs a{act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out, M, N, K, R, stream};
  if (format == GEMM_W4A4_FMT_NVFP4) return nv_run(variant, out_f16 == 1, a);
  if (format == GEMM_W4A4_FMT_MXFP4) return mx_run(variant, out_f16 == 1, a);
  return GEMM_W4A4_EINVAL;
}

extern "C" int gemm_w4a4_plan_variant(int format, int variant, int M, int N, int K, int R,
                                      gemm_w4a4_plan_t* plan) {
  if (format == GEMM_W4A4_FMT_NVFP4) return nv_plan(variant, M, N, K, R, plan);
  if (format == GEMM_W4A4_FMT_MXFP4) return mx_plan(variant, M, N, K, R, plan);
  return GEMM_W4A4_EINVAL;
}
