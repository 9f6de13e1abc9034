// gemm_w4a4.hip — fused NVFP4 W4A4 GEMM + per-column affine + rank-R LoRA for gfx950.
//
// y[m,n] = wcscale[n] * sum_k A[m,k] W[n,k] + bias[n] + sum_r la[m,r] lu[r,n]
// (operator and formats: the SVDQuant W4A4 on Blackwell page, sections 2, 3.1
// and 6.6; E2M1 bit layout: the DeepGEMM FP4 indexer page, "Step 0").
//
// Design (one workgroup per BM x BN output tile, WM x WN waves, 1 wave/SIMD):
//  * Loader: an LDS ring whose depth S the budget solver sets (3 or 4
//    stages; w4a4_layout.hpp). Each stage (128 values of k) of packed act and
//    wgt moves HBM -> LDS by direct-to-LDS DMA (global_load_lds), 16-byte
//    chunks XOR-swizzled by row so the consumer's LDS reads do not conflict.
//    The stage's E4M3 scale tiles are loaded by the workgroup with coalesced
//    8-byte loads (12-byte windows when M % 8 != 0), converted once to fp16
//    and stored [k-block][row] in LDS.
//    A stage's DMA is issued S-1 iterations before it is consumed.
//  * Decode: NVFP4 is exact in fp16. Every E2M1 value times every E4M3 scale
//    has at most 6 significant bits and lies in [2^-10, 2688], so each operand
//    value is built exactly as fp16: v_cvt_scalef32_pk_f16_fp4 (scale 1.0;
//    the instruction applies only the exponent of its scale operand, so the
//    E4M3 mantissa cannot ride on it) turns two nibbles into two fp16 values
//    and one packed fp16 multiply by the broadcast block scale applies the
//    scale.
//  * K-loop: v_mfma_f32_32x32x16_f16, whose 16-deep k-step is exactly one
//    NVFP4 scale block. Each lane feeds 8 values of k that share one scale.
//    The k <-> MFMA-slot assignment is free as long as both operands use the
//    same one (the sum over k does not depend on its order), so a lane takes
//    the 8 nibbles of one packed dword.
//  * Epilogue: acc = acc * wcscale[n] + bias[n] (one fp32 FMA); then the
//    LoRA-up product runs as further k-steps of the same-shape MFMA
//    (v_mfma_f32_32x32x16_bf16, identical accumulator layout) into the same
//    accumulators; then bf16 round-to-nearest-even, masked store of rows < M
//    and columns < N.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_w4a4.h"
#include "w4a4_common.hpp"
#include "w4a4_epilogue.hpp"
#include "w4a4_host.hpp"
#include "w4a4_layout.hpp"

namespace w4a4 {

// Eight E2M1 nibbles of one dword times the block scale (fp16 bits in half
// `half` of `scales`), as fp16. Which nibble lands in which of the eight slots is
// irrelevant (see the file comment); both operands go through this function.
__device__ __forceinline__ f16x8 decode8(uint32_t w, uint32_t scales, int half) {
  const _Float16 s = __builtin_bit_cast(f16x2, scales)[half];
  const f16x2 ss = {s, s};
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Eight E4M3 bytes -> eight fp16 (exact: every E4M3 value is zero, NaN or an
// fp16 normal number). The conversion applies only the exponent of its scale
// operand, and 1.0 has exponent 0.
__device__ __forceinline__ u32x4 e4m3x8_to_f16(u32x2 b) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 1.0f, true))};
}

// Eight scale bytes of k-block kb (clamped to the last one) for rows
// r0 .. r0+7 of a [KB][rows] tensor. `fast` (uniform over the workgroup) says
// the whole tile lies inside `rows` and rows are 8-byte aligned; otherwise each
// byte is read separately with its row clamped into range. The load itself is
// unconditional: k-blocks past K are zeroed where the scales are stored, so no
// register is written before the load returns.
__device__ __forceinline__ u32x2 load_scales8(const uint8_t* sc, int kb, int KB, int r0, int rows,
                                              bool fast) {
  const uint32_t base = uint32_t(min(kb, KB - 1)) * uint32_t(rows);
  if (fast) return *reinterpret_cast<const u32x2*>(sc + base + uint32_t(r0));
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = sc[base + uint32_t(min(r0 + i, rows - 1))];
    w[i >> 2] |= b << (8 * (i & 3));
  }
  return u32x2{w[0], w[1]};
}

// Scale bytes where rows of the scale tensor are not 8-byte aligned
// (M % 8 != 0): a 12-byte window of three dwords, loaded as it stands and
// reduced to the eight bytes only when the scales are stored, an iteration
// later, so no load result is waited for inside the K-loop. The tensor's base
// and its size must be multiples of 4 bytes (the host checks this), and the
// window start is clamped so that it never leaves the tensor: near the end the
// eight bytes then begin further into the window, and bytes the window does
// not hold belong to rows past `rows` (discarded outputs) only. Rows past
// `rows` read clamped addresses.
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
struct ScaleWindow {
  uint32_t start;   // byte offset of the window in the tensor (a multiple of 4)
  uint32_t pos;     // offset of the first of the eight bytes in the window, 0 .. 11
};
__device__ __forceinline__ ScaleWindow scale_window(int kb, int KB, int r0, int rows) {
  const uint32_t at = uint32_t(min(kb, KB - 1)) * uint32_t(rows) + uint32_t(min(r0, rows - 1));
  const uint32_t start = min(at & ~3u, uint32_t(KB) * uint32_t(rows) - 12u);
  return ScaleWindow{start, at - start};
}
__device__ __forceinline__ u32x2 window_bytes(u32x3_a4 v, uint32_t pos) {
  const uint32_t q = pos >> 2, sh = (pos & 3u) * 8u;
  const uint32_t a = q == 0 ? v.x : (q == 1 ? v.y : v.z);
  const uint32_t b = q == 0 ? v.y : v.z;
  return u32x2{__builtin_amdgcn_alignbit(b, a, sh), __builtin_amdgcn_alignbit(v.z, b, sh)};
}

// Two flavours per tile shape. The fast one (GENERAL = false) needs packed
// rows that are a multiple of 16 bytes (K % 32 == 0), N % 8 == 0, R % 8 == 0,
// 8-byte aligned wgt scales and 16-byte aligned LoRA operands: it moves packed
// data in 16-byte DMA pieces, scales in 8-byte loads (12-byte windows when
// M % 8 != 0) and LoRA operands in
// 16-byte loads, with no per-lane branches; ABYTE instantiates it with every
// scale read through a 12-byte window (scale_window), for act scales whose rows
// are not 8-byte aligned, so that aligned shapes run code without that path.
// The general one takes
// every valid shape: 4-byte DMA pieces (packed rows are always a multiple of
// 8 bytes), scales byte by byte at the edges, LoRA operands element by element.
// F16 selects the 16-bit type of the LoRA operands and of the output:
// IEEE binary16 (true) or bfloat16 (false); both round to nearest even.
// PART (fast flavour, K % 128 == 0): workgroup (tile, blockIdx.y) runs slice
// blockIdx.y of gridDim.y of the tile's K stages and stores float32 sums to
// p.part (see epilogue); split_k_reduce adds the slices.
template <class C, bool GENERAL, bool F16, bool ABYTE, bool PART = false>
__global__ __launch_bounds__(C::THREADS, C::OCC * C::THREADS / 256) void gemm_w4a4_kernel(
    const Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  constexpr int DMA_BYTES = GENERAL ? 4 : 16;
  constexpr int DMA_N = C::PACKED_BYTES / (C::THREADS * DMA_BYTES);   // DMA per thread per stage

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;                 // which half of the wave (k group)
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform copy (for M0)
  // wave = (wm * KG + kg) * WN + wn: k-group kg of wave tile (wm, wn)
  const int wn = wave % C::WN, wm = wave / C::WN / C::KG;
  const int kg = (wave_u / C::WN) % C::KG;   // uniform

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = (p.tm0 + tm) * C::BM, n0 = tn * C::BN;
  const int M = p.M, N = p.N;
  const int rowbytes = p.K >> 1;           // packed row stride
  // the stages [ks0, ks1) this workgroup runs: all, or its K slice; the
  // operand pointers start at the first of them
  static_assert(!PART || (!GENERAL && !ABYTE), "K slices run on the fast flavour");
  const int nst_all = (p.K + C::BK - 1) / C::BK;
  const int ks0 = PART ? int(blockIdx.y) * nst_all / int(gridDim.y) : 0;
  const int ks1 = PART ? (int(blockIdx.y) + 1) * nst_all / int(gridDim.y) : nst_all;
  const uint8_t* const act = p.act + (PART ? size_t(ks0) * C::ROW_BYTES : 0);
  const uint8_t* const wgt = p.wgt + (PART ? size_t(ks0) * C::ROW_BYTES : 0);
  const uint8_t* const ascales = p.ascales + (PART ? size_t(ks0) * C::KBLK * size_t(M) : 0);
  const uint8_t* const wscales = p.wscales + (PART ? size_t(ks0) * C::KBLK * size_t(N) : 0);
  const int K = PART ? (ks1 - ks0) * C::BK : p.K;   // k of this workgroup
  const int kbytes = K >> 1;               // packed bytes of a row it reads
  const int KB = K >> 4;                   // scale blocks along k
  const int nst = (K + C::BK - 1) / C::BK;

  // ---- DMA sources. LDS slot q (DMA_BYTES each) of a stage's packed region,
  // q = u*THREADS + tid, holds for row = byte/64, swizzled chunk position cp
  // and piece pc, the bytes of data chunk cp ^ swz(row). A round u moves
  // THREADS*DMA_BYTES/64 whole rows, so the row of slot q is the row of round 0
  // plus u*ROWS_PER_ROUND. The swizzle repeats every 32 rows; when a round is a
  // multiple of 32 rows the offset inside the row is the same in every round,
  // otherwise (4-byte pieces) it is recomputed per round.
  static_assert(C::B_OFF % (C::THREADS * DMA_BYTES) == 0, "DMA rounds must not straddle A/B");
  constexpr int ROWS_PER_ROUND = C::THREADS * DMA_BYTES / C::ROW_BYTES;
  constexpr bool SAME_INROW = ROWS_PER_ROUND % 32 == 0;
  constexpr int A_ROUNDS = C::B_OFF / (C::THREADS * DMA_BYTES);
  const int dma_row0 = tid * DMA_BYTES / C::ROW_BYTES;
  const int dma_cp = (tid * DMA_BYTES / 16) & 3;
  const int dma_pc = (tid * DMA_BYTES % 16) / DMA_BYTES;
  const uint32_t dma_inrow = uint32_t(((dma_cp ^ swz(dma_row0)) * 16) + dma_pc * DMA_BYTES);
  const bool dma_a_inside = m0 + C::BM <= M, dma_b_inside = n0 + C::BN <= N;
  const uint32_t dma_a0 = uint32_t(m0 + dma_row0) * uint32_t(rowbytes) + dma_inrow;
  const uint32_t dma_b0 = uint32_t(n0 + dma_row0) * uint32_t(rowbytes) + dma_inrow;
  const uint32_t dma_round = uint32_t(ROWS_PER_ROUND) * uint32_t(rowbytes);

  const int full_stages = kbytes / C::ROW_BYTES;   // stages lying entirely inside K
  // Round u of stage `st`'s packed bytes into ring slot `buf` % STAGES.
  auto dma_part = [&](int st, int buf, int u) __attribute__((always_inline)) {
    uint8_t* stage = smem + (buf % C::STAGES) * C::STAGE_BYTES;
    const uint32_t k0 = uint32_t(st * C::ROW_BYTES);
    // pieces past the row end (partial last stage only) re-read the row's
    // first piece; their k-blocks get a zero scale
    const bool tail_stage = st >= full_stages;
    {
      const bool is_b = u >= A_ROUNDS;
      const int ur = is_b ? u - A_ROUNDS : u;
      const uint32_t inrow =
          SAME_INROW ? dma_inrow
                     : uint32_t(((dma_cp ^ swz(dma_row0 + ur * ROWS_PER_ROUND)) * 16) +
                                dma_pc * DMA_BYTES);
      const bool tail = tail_stage && inrow + k0 + DMA_BYTES > uint32_t(kbytes);
      const uint32_t kin = tail ? 0u : k0 + inrow;
      uint32_t row_off;
      if (is_b ? dma_b_inside : dma_a_inside) {
        row_off = (is_b ? dma_b0 : dma_a0) - dma_inrow + uint32_t(ur) * dma_round;
      } else {   // edge tile: rows past M or N are clamped into range
        const int row = (is_b ? n0 : m0) + dma_row0 + ur * ROWS_PER_ROUND;
        row_off = uint32_t(min(row, (is_b ? N : M) - 1)) * uint32_t(rowbytes);
      }
      const uint8_t* src = (is_b ? wgt : act) + (row_off + kin);
      dma<DMA_BYTES>(src, stage + (u * C::THREADS + wave_u * 64) * DMA_BYTES);
    }
  };
  auto issue_dma = [&](int st, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < DMA_N; ++u) dma_part(st, buf, u);
  };

  // ---- scale loader. Thread t < SA_THREADS owns rows r8 .. r8+7 of the act
  // scales for k-block pair kp (k-blocks 2kp, 2kp+1 of the stage); the next
  // SB_THREADS threads do the same for wgt; the rest load nothing.
  const bool s_is_a = tid < C::SA_THREADS;
  const bool s_is_b = !s_is_a && tid < C::SA_THREADS + C::SB_THREADS;
  const int s_idx = s_is_a ? tid : tid - C::SA_THREADS;
  const int s_rows8 = (s_is_a ? C::BM : C::BN) / 8;
  const int s_kp = s_idx / s_rows8;
  const int s_r8 = (s_idx % s_rows8) * 8;
  const uint8_t* s_src = s_is_a ? ascales : wscales;
  const int s_rows = s_is_a ? M : N;
  const int s_r0 = (s_is_a ? m0 : n0) + s_r8;
  const int s_off = (s_is_a ? C::SA_OFF : C::SB_OFF) +
                    (s_kp * (s_is_a ? C::BM : C::BN) + s_r8) * 4;
  // 8-byte scale loads need the whole tile in range and 8-aligned rows
  const bool s_fast = s_is_a ? ((M & 7) == 0 && (reinterpret_cast<uintptr_t>(p.ascales) & 7u) == 0 &&
                                m0 + C::BM <= M)
                             : ((N & 7) == 0 && (reinterpret_cast<uintptr_t>(p.wscales) & 7u) == 0 &&
                                n0 + C::BN <= N);
  // raw scale bytes (two k-blocks) of one stage: [0] in the loop, [1] too in the prologue
  // (ABYTE: 12-byte windows, see scale_window; both scale tensors, so that no
  // thread branches on its role)
  using RawT = std::conditional_t<ABYTE, u32x3_a4, u32x2>;
  RawT s_raw[2][2] = {};

  auto load_scale_half = [&](int st, RawT (&raw)[2], int e) __attribute__((always_inline)) {
    const int kb = st * C::KBLK + 2 * s_kp + e;
    if constexpr (!GENERAL) {
      // rows % 8 == 0 and 8-byte aligned scales: a group of 8 rows is wholly
      // inside or wholly past the edge, where it re-reads the last group (its
      // rows only reach discarded outputs). Threads without a scale role read
      // a clamped address too and store nothing, so this load is unconditional.
      if constexpr (ABYTE) {
        raw[e] = *reinterpret_cast<const u32x3_a4*>(s_src + scale_window(kb, KB, s_r0, s_rows).start);
      } else {
        raw[e] = *reinterpret_cast<const u32x2*>(s_src + uint32_t(min(kb, KB - 1)) * uint32_t(s_rows) +
                                                 uint32_t(min(s_r0, s_rows - 8)));
      }
    } else {
      if (s_is_a || s_is_b) raw[e] = load_scales8(s_src, kb, KB, s_r0, s_rows, s_fast);
    }
  };
  auto load_scales = [&](int st, RawT (&raw)[2]) __attribute__((always_inline)) {
    load_scale_half(st, raw, 0);
    load_scale_half(st, raw, 1);
  };
  // k-blocks past K get scale 0: their packed bytes (re-read from the row
  // start) then contribute exactly zero, since E2M1 values are finite.
  // Stored interleaved: row r of pair kp holds (scale of 2kp, scale of 2kp+1).
  auto store_scales = [&](int st, int buf, const RawT (&raw)[2]) __attribute__((always_inline)) {
    if (s_is_a || s_is_b) {
      const int kb = st * C::KBLK + 2 * s_kp;
      const u32x2 zero = {0u, 0u};
      u32x2 b0, b1;
      if constexpr (ABYTE) {
        b0 = window_bytes(raw[0], scale_window(kb, KB, s_r0, s_rows).pos);
        b1 = window_bytes(raw[1], scale_window(kb + 1, KB, s_r0, s_rows).pos);
      } else {
        b0 = raw[0];
        b1 = raw[1];
      }
      const u32x4 h0 = e4m3x8_to_f16(kb < KB ? b0 : zero);
      const u32x4 h1 = e4m3x8_to_f16(kb + 1 < KB ? b1 : zero);
      uint8_t* dst = smem + (buf % C::STAGES) * C::STAGE_BYTES + s_off;
      const u32x4 lo = {__builtin_amdgcn_perm(h1.x, h0.x, 0x05040100u),
                        __builtin_amdgcn_perm(h1.x, h0.x, 0x07060302u),
                        __builtin_amdgcn_perm(h1.y, h0.y, 0x05040100u),
                        __builtin_amdgcn_perm(h1.y, h0.y, 0x07060302u)};
      const u32x4 hi = {__builtin_amdgcn_perm(h1.z, h0.z, 0x05040100u),
                        __builtin_amdgcn_perm(h1.z, h0.z, 0x07060302u),
                        __builtin_amdgcn_perm(h1.w, h0.w, 0x05040100u),
                        __builtin_amdgcn_perm(h1.w, h0.w, 0x07060302u)};
      *reinterpret_cast<u32x4*>(dst) = lo;
      *reinterpret_cast<u32x4*>(dst + 16) = hi;
    }
  };

  // ---- per-lane LDS read offsets (relative to a stage). Lane (row l32,
  // half g) of MFMA tile i reads row r = wm*TM + 32i + l32, bytes 32g .. 32g+31
  // of the stage: data chunk 2g (k-steps 0-3) and 2g+1 (k-steps 4-7); k-step s
  // uses dword s & 3 of chunk s >> 2. Its scales are k-blocks 4g .. 4g+3,
  // pairs 2g (chunk 0) and 2g+1 (chunk 1). Rows 32 apart have the same
  // swizzle, so tile i's offsets are tile 0's plus the constant i*32 rows.
  const int ra = wm * C::TM + l32, rb = wn * C::TN + l32;
  const uint32_t a_rd0 = C::A_OFF + ra * C::ROW_BYTES + (((2 * g) ^ swz(ra)) << 4);
  const uint32_t b_rd0 = C::B_OFF + rb * C::ROW_BYTES + (((2 * g) ^ swz(rb)) << 4);
  const uint32_t sa_rd0 = C::SA_OFF + (2 * g * C::BM + ra) * 4;
  const uint32_t sb_rd0 = C::SB_OFF + (2 * g * C::BN + rb) * 4;

  // One 16-byte chunk (4 k-steps) of this lane's operands and its two block
  // scales, both in one register (one 4-byte LDS read; the packed fp16
  // multiply broadcasts either half for free).
  struct Chunk {
    u32x4 a[C::MI], b[C::NI];
    uint32_t sa[C::MI], sb[C::NI];   // fp16 scales of the chunk's two k-block pairs
  };
  // Tile t (act tiles 0 .. MI-1, then wgt tiles) of chunk h of stage st.
  auto read_tile = [&](int st, int h, int t, Chunk& R) __attribute__((always_inline)) {
    const uint8_t* stage = smem + (st % C::STAGES) * C::STAGE_BYTES;
    // chunk 2g+1 sits at chunk position ((2g) ^ swz) ^ 1: flip bit 4
    if (t < C::MI) {
      const uint8_t* pa = stage + (h ? (a_rd0 ^ 16u) : a_rd0);
      const uint32_t* qa = reinterpret_cast<const uint32_t*>(stage + sa_rd0 + h * C::BM * 4);
      R.a[t] = *reinterpret_cast<const u32x4*>(pa + t * 32 * C::ROW_BYTES);
      R.sa[t] = qa[t * 32];
    } else {
      const int j = t - C::MI;
      const uint8_t* pb = stage + (h ? (b_rd0 ^ 16u) : b_rd0);
      const uint32_t* qb = reinterpret_cast<const uint32_t*>(stage + sb_rd0 + h * C::BN * 4);
      R.b[j] = *reinterpret_cast<const u32x4*>(pb + j * 32 * C::ROW_BYTES);
      R.sb[j] = qb[j * 32];
    }
  };
  auto read_chunk = [&](int st, int h, Chunk& R) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < C::MI + C::NI; ++t) read_tile(st, h, t, R);
  };

  // acc[j][i] is the 32x32 tile D[n][m] = sum_k W[n,k] A[m,k] (wgt as the
  // MFMA's A operand, act as its B operand): lane (l32, g) holds column
  // m = 32i + l32 and, in element 4q + t, row n = 32j + 8q + 4g + t, i.e. four
  // consecutive output columns of one output row.
  f32x16 acc[C::NI][C::MI];
#pragma unroll
  for (int j = 0; j < C::NI; ++j)
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // ---- decode software-pipelined one k-step ahead of the MFMAs. D[p] holds
  // the decoded operands of the k-steps of parity p. k-step s of a chunk uses
  // dword s and scale s >> 1 of every tile. The 12 MFMAs of one k-step are
  // issued one per group, each followed by at most one tile decode (8 VALU)
  // for the next k-step; a scheduling fence closes every group. The VALU work
  // then runs in the shadow of the MFMA just issued instead of piling up
  // between MFMAs, which a single wave per SIMD cannot hide.
  struct Dec {
    f16x8 a[C::MI], b[C::NI];
  };
  Dec D[2];
  auto decode_tile = [&](int t, const Chunk& R, int s, Dec& d) __attribute__((always_inline)) {
    if (t < C::MI)
      d.a[t] = decode8(R.a[t][s], R.sa[t], s >> 1);
    else
      d.b[t - C::MI] = decode8(R.b[t - C::MI][s], R.sb[t - C::MI], s >> 1);
  };
  // Pair p (0 .. 4T-1) of a k-step: the two fp16 values 2h, 2h+1 of tile
  // t = p / 4, h = p % 4 (one conversion and one packed multiply).
  auto decode_pair = [&](int pr, const Chunk& R, int s, Dec& d) __attribute__((always_inline)) {
    const int t = pr / 4, h = pr % 4;
    const uint32_t w = t < C::MI ? R.a[t][s] : R.b[t - C::MI][s];
    const uint32_t sc = t < C::MI ? R.sa[t] : R.sb[t - C::MI];
    const _Float16 sv = __builtin_bit_cast(f16x2, sc)[s >> 1];
    f16x2 c;
    switch (h) {   // the word select must be an immediate; folds after unrolling
      case 0: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0); break;
      case 1: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1); break;
      case 2: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2); break;
      default: c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3); break;
    }
    const f16x2 v = c * f16x2{sv, sv};
    f16x8& o = t < C::MI ? d.a[t] : d.b[t - C::MI];
    o[2 * h] = v[0];
    o[2 * h + 1] = v[1];
  };
  auto decode_all = [&](const Chunk& R, int s, Dec& d) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < C::MI + C::NI; ++t) decode_tile(t, R, s, d);
  };
  // ---- pipeline over an S-deep LDS ring (S = C::STAGES >= 3). Iteration st
  // computes stage st, DMAs stage st+S-1, loads the raw scales of stage st+2
  // (register set st % 2), stores the fp16 scales of stage st+1 (loaded one
  // iteration earlier, set (st+1) % 2) into its buffer, and reads chunk 1 of
  // stage st and chunk 0 of stage st+1 into registers. The one barrier sits in
  // the middle of the iteration, right before the first read of stage st+1:
  // it publishes stage st+1 (DMA and scales), and every read of stage st-1
  // (its chunk 1 is read in k-steps 0-2 of iteration st-1) happened before the
  // previous one, so DMA(st+S-1) may refill buffer (st+S-1) % S = (st-1) % S
  // from the start of iteration st. The prologue issues DMA(0 .. S-2) and only
  // waits for stage 0; stage 1 has three k-steps of stage 0's compute to
  // arrive in.
  //
  // Prefetches past the last stage read clamped, in-range addresses into
  // buffers nobody reads again, and stages past K get zero scales, which keeps
  // the loop body free of branches. Vector-memory ops complete in issue
  // order: the prologue issues SCL(0), DMA(0), SCL(1), DMA(1 .. S-2), and
  // iteration j issues SCL(j+2) then DMA(j+S-1). The scale store of iteration
  // st needs SCL(st+1) and DMA(st+1). With S >= 4, DMA(st+1) is older than
  // SCL(st+1), and the ops issued after SCL(st+1) are DMA(st+S-2), SCL(st+2)
  // and DMA(st+S-1); with S = 3, DMA(st+1) is the younger one and SCL(st+2),
  // DMA(st+2) follow it. Waiting until at most min(S-2, 2) DMA rounds plus one
  // scale load pair remain completes both (for st = 0 more may remain; the
  // smaller count is the stricter wait and serves every st).
  //
  // Inside an iteration every instruction has a fixed slot: k-step S (0..7)
  // runs G MFMA groups; group q issues MFMA q, decodes
  // pairs [4Tq/G, 4T(q+1)/G) of the next k-step's decode (the conversion
  // issues at half rate, so the decode is spread evenly over all groups),
  // and issues the memory op of slot S*G + q, if any:
  //   slots 0, 1                scale loads of stage st+2 (two k-blocks)
  //   slots 2 .. 2+DMA_SLOTS-1  DMA rounds of stage st+3 (one per slot; the
  //                             general flavour's many 4-byte rounds at once)
  //   next T slots              tiles of chunk 1 of stage st (decoded from k-step 3 on)
  //   slot SLOT_SCL (k-step 3)  fp16 scales of stage st+1 into its buffer
  //   slot 4G (k-step 4)        the barrier, after that group's MFMA
  //   slots 4G .. 4G+T-1        tiles of chunk 0 of stage st+1 (decoded in k-step 7)
  // A scheduling fence closes every group, so no memory op or decode bunches
  // up between two MFMAs: one wave per SIMD keeps its MFMA pipe fed.
  constexpr int G = C::MI * C::NI;
  constexpr int T = C::MI + C::NI;
  constexpr int DMA_SLOTS = GENERAL ? 1 : DMA_N, DMA_PER_SLOT = DMA_N / DMA_SLOTS;
  constexpr int SLOT_RD1 = 2 + DMA_SLOTS, SLOT_RD0 = 4 * G, SLOT_SCL = 3 * G + G / 2;
  // ops issued after SCL(st+1): DMA(st+2), SCL(st+2) (2 loads per thread in
  // the fast flavour; the general one counts none, which waits longer), DMA(st+3)
  constexpr int VM_AFTER_SCL = std::min(C::STAGES - 2, 2) * DMA_N + (GENERAL ? 0 : 2);
  static_assert(VM_AFTER_SCL < 64, "vmcnt range");
  static_assert(T <= G, "one decode per MFMA group");
  static_assert(SLOT_RD1 + T <= 3 * G, "chunk 1 must be requested before k-step 3 decodes it");
  static_assert(SLOT_RD1 + T <= SLOT_SCL, "slots overlap");
  const int last = nst - 1;
  Chunk C0, C1;
  EpiRegs epi_regs;
  // DEEP (KG == 2, fast flavours): raw scales of stage j in set j % 4,
  // loaded with the DMA of the same stage (S-1 stages ahead: a k-group
  // iteration is a quarter of a single-group one, too short to cover a load
  // issued one stage ahead). The general flavour keeps the single-group
  // prefetch (the deeper one's unrolling costs it scalar registers).
  constexpr bool DEEP = C::KG == 2 && !GENERAL;
  RawT s_raw4[DEEP ? 4 : 1][2] = {};
  epilogue_prefetch<C, GENERAL>(p, smem, tid, m0, n0, epi_regs);   // older than every ring op below
  if constexpr (!DEEP) {
    load_scales(0, s_raw[0]);
    issue_dma(0, 0);
    load_scales(min(1, last), s_raw[1]);
#pragma unroll
    for (int j = 1; j < C::STAGES - 1; ++j) issue_dma(min(j, last), j);
    // SCL(0), DMA(0): after them come SCL(1) and DMA(1 .. S-2)
    wait_vm_lgkm0<std::min(63, (C::STAGES - 2) * DMA_N + (GENERAL ? 0 : 2))>();
    store_scales(0, 0, s_raw[0]);
  } else {
    static_assert(C::STAGES <= 4, "scale sets cover S-1 stages ahead");
#pragma unroll
    for (int j = 0; j < C::STAGES - 1; ++j) {
      load_scales(min(j, last), s_raw4[j]);
      issue_dma(min(j, last), j);
    }
    // SCL(0), DMA(0): after them come SCL(j), DMA(j) for j = 1 .. S-2
    wait_vm_lgkm0<std::min(63, (C::STAGES - 2) * (DMA_N + (GENERAL ? 0 : 2)))>();
    store_scales(0, 0, s_raw4[0]);
  }
  wait_vm_lgkm0<63>();
  wg_barrier();
  read_chunk(0, kg, C0);   // KG == 1: chunk 0; KG == 2: the k-group's own chunk
  decode_all(C0, 0, D[0]);

  // PAR = st & 1, fixed per call site of the two-way unrolled loop.
  auto iteration = [&]<int PAR>(int st) __attribute__((always_inline)) {
    const int st_scl = min(st + 2, last), st_dma = min(st + C::STAGES - 1, last);
    // k-step S: Sv is an int, or (general flavour) a std::integral_constant
    auto kstep = [&](auto Sv) __attribute__((always_inline)) {
      const int S = Sv;
      const Dec& cur = D[S & 1];
      Dec& nxt = D[(S + 1) & 1];
      const Chunk& Rn = (S + 1 >= 4 && S + 1 < 8) ? C1 : C0;
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int j = q / C::MI, i = q % C::MI;
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.b[j], cur.a[i], acc[j][i], 0, 0, 0);
        const int slot = S * G + q;
        if (slot == SLOT_RD0) {
          wait_vm_lgkm0<63>();   // this wave's scale stores
          wg_barrier();
        }
#pragma unroll
        for (int pr = 4 * T * q / G; pr < 4 * T * (q + 1) / G; ++pr) decode_pair(pr, Rn, (S + 1) & 3, nxt);
        if (slot < 2)
          load_scale_half(st_scl, s_raw[PAR], slot);
        else if (slot < SLOT_RD1)
#pragma unroll
          for (int u = 0; u < DMA_PER_SLOT; ++u)
            dma_part(st_dma, st + C::STAGES - 1, (slot - 2) * DMA_PER_SLOT + u);
        else if (slot < SLOT_RD1 + T)
          read_tile(st, 1, slot - SLOT_RD1, C1);
        else if (slot == SLOT_SCL) {
          wait_vm<VM_AFTER_SCL>();
          store_scales(st + 1, st + 1, s_raw[1 - PAR]);   // unclamped: stages past K get zero scales
        } else if (slot >= SLOT_RD0 && slot < SLOT_RD0 + T)
          read_tile(st + 1, 0, slot - SLOT_RD0, C0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // The general flavour's branches keep the compiler from resolving the
    // chunk and decode-buffer choices of a runtime k-step index, which then
    // leaves those arrays in scratch memory; a compile-time index avoids it.
    // The fast flavour schedules slightly better from the plain loop.
    if constexpr (GENERAL) {
      static_for<0, 8>([&]<int S>() __attribute__((always_inline)) { kstep(std::integral_constant<int, S>{}); });
    } else {
#pragma unroll
      for (int S = 0; S < 8; ++S) kstep(S);
    }
  };
  // ---- KG == 2: k-group kg runs k-steps 4kg .. 4kg+3 of every stage, from
  // chunk kg of its operand rows, 4 k-steps of G MFMA groups per iteration.
  // The memory ops keep the order and waits of the single-group schedule:
  // slots 0, 1 scale loads of stage st+2, then the DMA rounds of stage st+S-1,
  // slot SLOT_SCL2 the fp16 scales of stage st+1, slot SLOT_RD2 (k-step 2)
  // the barrier that publishes stage st+1, then the k-group's T tiles of
  // stage st+1 (decoded in k-step 3). The k-group reads nothing else, so
  // every read of stage st-1 precedes the barrier of iteration st-1, and
  // DMA(st+S-1) may refill its buffer from the start of iteration st.
  constexpr int SLOT_SCL2 = G + G / 2, SLOT_RD2 = 2 * G;
  // ops issued after DMA(st+1) when stage st+1's scales are stored: the S-2
  // later pairs SCL(j), DMA(j) (the general flavour counts no scale loads,
  // which waits longer); SCL(st+1) precedes DMA(st+1)
  constexpr int VM_KG = DEEP ? std::min(63, (C::STAGES - 2) * (DMA_N + 2)) : VM_AFTER_SCL;
  auto iteration_kg = [&]<int PAR>(int st) __attribute__((always_inline)) {
    // stage st's chunk is in C0 for even st, C1 for odd; stage st+1's goes to the other
    Chunk& Cc = *[&]() { if constexpr (PAR % 2 == 0) return &C0; else return &C1; }();
    Chunk& Cn = *[&]() { if constexpr (PAR % 2 == 0) return &C1; else return &C0; }();
    // scales: DEEP loads stage st+S-1 into set (st+S-1) % 4 and stores stage
    // st+1 from set (st+1) % 4; otherwise stage st+2 into s_raw[st % 2], as
    // the single-group loop
    RawT (&sc_load)[2] = *[&]() { if constexpr (DEEP) return &s_raw4[(PAR + C::STAGES - 1) % 4]; else return &s_raw[PAR % 2]; }();
    RawT (&sc_store)[2] = *[&]() { if constexpr (DEEP) return &s_raw4[(PAR + 1) % 4]; else return &s_raw[1 - PAR % 2]; }();
    const int st_scl = min(st + (DEEP ? C::STAGES - 1 : 2), last);
    const int st_dma = min(st + C::STAGES - 1, last);
    auto kstep = [&](auto Sv) __attribute__((always_inline)) {
      const int S = Sv;
      const Dec& cur = D[S & 1];
      Dec& nxt = D[(S + 1) & 1];
      const Chunk& Rn = S + 1 < 4 ? Cc : Cn;
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int j = q / C::MI, i = q % C::MI;
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.b[j], cur.a[i], acc[j][i], 0, 0, 0);
        const int slot = S * G + q;
        if (slot == SLOT_RD2) {
          wait_vm_lgkm0<63>();   // this wave's scale stores
          wg_barrier();
        }
#pragma unroll
        for (int pr = 4 * T * q / G; pr < 4 * T * (q + 1) / G; ++pr) decode_pair(pr, Rn, (S + 1) & 3, nxt);
        if (slot < 2)
          load_scale_half(st_scl, sc_load, slot);
        else if (slot < SLOT_RD1)
#pragma unroll
          for (int u = 0; u < DMA_PER_SLOT; ++u)
            dma_part(st_dma, st + C::STAGES - 1, (slot - 2) * DMA_PER_SLOT + u);
        else if (slot == SLOT_SCL2) {
          wait_vm<VM_KG>();
          store_scales(st + 1, st + 1, sc_store);
        } else if (slot >= SLOT_RD2 && slot < SLOT_RD2 + T)
          read_tile(st + 1, kg, slot - SLOT_RD2, Cn);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (GENERAL) {
      static_for<0, 4>([&]<int S>() __attribute__((always_inline)) { kstep(std::integral_constant<int, S>{}); });
    } else {
#pragma unroll
      for (int S = 0; S < 4; ++S) kstep(S);
    }
  };

  int st = 0;
  if constexpr (C::KG == 1) {
    for (; st + 1 < nst; st += 2) {
      iteration.template operator()<0>(st);
      iteration.template operator()<1>(st + 1);
    }
    if (st < nst) iteration.template operator()<0>(st);
  } else {
    static_assert(C::KG == 2, "one or two k-groups");
    static_assert(SLOT_RD1 <= SLOT_SCL2 && SLOT_SCL2 < SLOT_RD2 && SLOT_RD2 + T <= 3 * G,
                  "k-group schedule: scales, DMA, scale store, barrier, then the next stage's chunk");
    if constexpr (DEEP) {
      for (; st + 3 < nst; st += 4) {
        iteration_kg.template operator()<0>(st);
        iteration_kg.template operator()<1>(st + 1);
        iteration_kg.template operator()<2>(st + 2);
        iteration_kg.template operator()<3>(st + 3);
      }
      if (st < nst) iteration_kg.template operator()<0>(st);
      if (st + 1 < nst) iteration_kg.template operator()<1>(st + 1);
      if (st + 2 < nst) iteration_kg.template operator()<2>(st + 2);
    } else {
      for (; st + 1 < nst; st += 2) {
        iteration_kg.template operator()<0>(st);
        iteration_kg.template operator()<1>(st + 1);
      }
      if (st < nst) iteration_kg.template operator()<0>(st);
    }
  }
  wait_vm_lgkm0<0>();   // drain the prefetches past the last stage

  if constexpr (C::KG == 1) {
    epilogue<C, GENERAL, F16, PART>(acc, p, smem, tid, m0, n0, epi_regs);
  } else {
    // k-group kg keeps m-tiles [kg MIH, (kg+1) MIH) of the wave tile and adds
    // its partner's partial sums of them; it hands the other half to the
    // partner. Through the drained ring: wave w's outgoing tiles at
    // [w][tile][quarter][lane] (16 bytes per lane, consecutive lanes
    // consecutive: no bank conflicts).
    constexpr int MIH = C::MI / 2;
    using E = EpiView<C>;
    f32x16 kept[C::NI][MIH];
    const int partner = wave + (kg == 0 ? C::WN : -C::WN);
    float* xbuf = reinterpret_cast<float*>(smem);
    constexpr int TILE_F = 16 * kWave;   // floats per exchanged tile
    static_assert(C::THREADS / kWave * C::NI * MIH * TILE_F * 4 <= C::RING_BYTES, "exchange fits the ring");
    auto exchange = [&]<int KGC>() __attribute__((always_inline)) {
      f32x4* out = reinterpret_cast<f32x4*>(xbuf + wave * (C::NI * MIH * TILE_F));
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int ii = 0; ii < MIH; ++ii) {
          const f32x16& a = acc[j][(1 - KGC) * MIH + ii];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            out[((j * MIH + ii) * 4 + qq) * kWave + lane] = f32x4{a[4 * qq], a[4 * qq + 1], a[4 * qq + 2], a[4 * qq + 3]};
        }
      __syncthreads();
      const f32x4* in = reinterpret_cast<const f32x4*>(xbuf + partner * (C::NI * MIH * TILE_F));
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int ii = 0; ii < MIH; ++ii) {
          const f32x16& a = acc[j][KGC * MIH + ii];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x4 b = in[((j * MIH + ii) * 4 + qq) * kWave + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) kept[j][ii][4 * qq + e] = a[4 * qq + e] + b[e];
          }
        }
    };
    __syncthreads();   // every wave is done with the ring
    if (kg == 0) exchange.template operator()<0>();
    else exchange.template operator()<1>();
    __syncthreads();   // the epilogue reuses the ring
    epilogue<E, GENERAL, F16, PART>(kept, p, smem, tid, m0, n0, epi_regs);
  }
}

// ------------------------------------------------------------------ host side

template <class C>
VariantDesc nv_variant(double cost) {
  static const void* const k[2][3] = {
      {reinterpret_cast<const void*>(gemm_w4a4_kernel<C, true, false, false>),
       reinterpret_cast<const void*>(gemm_w4a4_kernel<C, false, false, false>),
       reinterpret_cast<const void*>(gemm_w4a4_kernel<C, false, false, true>)},
      {reinterpret_cast<const void*>(gemm_w4a4_kernel<C, true, true, false>),
       reinterpret_cast<const void*>(gemm_w4a4_kernel<C, false, true, false>),
       reinterpret_cast<const void*>(gemm_w4a4_kernel<C, false, true, true>)}};
  return describe<C>(k, true, cost);
}

// Relative costs per output element of a full round of tiles, measured on
// MI355X (bench.py --calibrate: every instance timed at each shape, time over
// rounds x tiles on the busiest CU x tile elements, relative to 256x192;
// medians over the four M = 4352 shapes, where every instance needs whole or
// nearly whole rounds): 256x128 1.16; the two 128x128 instances (two tiles
// per CU) 1.31 with a 4-deep ring and no side region, 1.30 with a 3-deep ring
// and the whole side region (the first LoRA chunk and wcscale/bias arrive
// during the K-loop); 64x192 with two k-groups 1.46-1.62, set to 1.55, which
// also reproduces its measured loss to 256x128 at 2000x3072x3072 (two of its
// rounds against one). Smaller wave tiles decode more operand tiles per MFMA
// (0.58 for 256x192, 0.75, 1.0, 0.83). tests/test_gpu_solver.py times every
// instance at shapes where the choice matters and requires the pick to be
// within 15 % of the fastest, so a kernel change that moves a cost far from
// its entry here fails there.
static const VariantDesc kVariants[] = {nv_variant<Cfg256x192>(1.00), nv_variant<Cfg128x128>(1.31),
                                        nv_variant<Cfg256x128>(1.16), nv_variant<Cfg128x128S>(1.30),
                                        nv_variant<Cfg64x192K>(1.55)};
static constexpr int kNumVariants = int(sizeof(kVariants) / sizeof(kVariants[0]));
// What a launch costs besides its k-loop, in k-stages of a full round of
// 256x192 tiles: a 4096x3072 launch over one stage (K = 128) takes about
// 11.7 us against 2.14 us per added stage.
static constexpr double kLaunchStages = 4.4;
// The instance compiled with K-sliced workgroups (the 64x192 k-group tile),
// as the tail of a split plan, and those kernels [F16].
static constexpr int kPartVariant = 4;
static const void* const kPartKernel[2] = {
    reinterpret_cast<const void*>(gemm_w4a4_kernel<Cfg64x192K, false, false, false, true>),
    reinterpret_cast<const void*>(gemm_w4a4_kernel<Cfg64x192K, false, true, false, true>)};
static const void* const kReduceKernel[2] = {reinterpret_cast<const void*>(split_k_reduce<false>),
                                             reinterpret_cast<const void*>(split_k_reduce<true>)};
// K slices need the fast flavour with 8-row act scales and whole stages.
static bool slices_ok(int M, int N, int K, int R) {
  return K % 128 == 0 && N % 8 == 0 && M % 8 == 0 && (R == 0 || R % 8 == 0);
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

// Flavour: fast where packed rows, wgt scales and LoRA operands allow wide
// accesses; within it, act scales in 8-byte loads when their rows are
// 8-byte aligned, else in 12-byte windows (needs a 4-byte aligned act-scale
// tensor of a multiple of 4 bytes, at least 12); general otherwise.
static int nv_flavour(int M, int N, int K, int R, uintptr_t ascales, uintptr_t wscales, uintptr_t lora) {
  const bool fast = K % 32 == 0 && N % 8 == 0 && (wscales & 7u) == 0 &&
                    (R == 0 || (R % 8 == 0 && (lora & 15u) == 0));
  const size_t a_bytes = size_t(K) / 16 * size_t(M);
  const bool a_rows8 = M % 8 == 0 && (ascales & 7u) == 0;
  const bool a_window = (ascales & 3u) == 0 && a_bytes % 4 == 0 && a_bytes >= 12;
  return !fast ? 0 : a_rows8 ? 1 : a_window ? 2 : 0;
}

int nv_plan(int variant, int M, int N, int K, int R, gemm_w4a4_plan_t* pl) {
  if (!pl || !sizes_ok(M, N, K, R) || variant < -1 || variant >= kNumVariants) return GEMM_W4A4_EINVAL;
  const Choice c = variant >= 0 ? Choice{variant, -1, M, 1}
                                 : choose_plan(kVariants, kNumVariants, M, N, K, kLaunchStages,
                                               slices_ok(M, N, K, R) ? kPartVariant : -1);
  const int rc = plan_choice(kVariants, c, M, N, K, R, pl);
  if (rc == GEMM_W4A4_OK) fill_registers(kVariants[c.main], nv_flavour(M, N, K, R, 0, 0, 0), pl);
  return rc;
}

int nv_run(int variant, bool f16, const CallArgs& a) {
  if (!sizes_ok(a.M, a.N, a.K, a.R) || variant < -1 || variant >= kNumVariants) return GEMM_W4A4_EINVAL;
  int rc = check_call(a, 16);
  if (rc != GEMM_W4A4_OK) return rc;
  gemm_w4a4_plan_t pl;
  if (nv_plan(variant, a.M, a.N, a.K, a.R, &pl) != GEMM_W4A4_OK) return GEMM_W4A4_EINVAL;
  rc = check_device();
  if (rc != GEMM_W4A4_OK) return rc;
  const int flavour = nv_flavour(a.M, a.N, a.K, a.R, uintptr_t(a.ascales), uintptr_t(a.wscales),
                                 a.R > 0 ? (uintptr_t(a.lora_act_in) | uintptr_t(a.lora_up)) : 0u);
  auto sliced = [&](int rows, int splits, int row0) -> int {
    // the fast flavour with 8-row act scales (flavour 1), and 16-byte aligned
    // float32 sums in the output
    if (flavour != 1 || (uintptr_t(a.out) & 15u) != 0) return GEMM_W4A4_EINVAL;
    return launch_slices(kPartKernel[f16 ? 1 : 0], kReduceKernel[f16 ? 1 : 0], kVariants[kPartVariant], rows, splits,
                         row0, a);
  };
  return launch_plan(kVariants, pl, a, [&](const VariantDesc& v) { return v.kernel[f16 ? 1 : 0][flavour]; }, sliced);
}

}  // namespace w4a4

using namespace w4a4;

extern "C" int gemm_w4a4_plan(int M, int N, int K, int R, gemm_w4a4_plan_t* plan) {
  return nv_plan(-1, M, N, K, R, plan);
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
    case GEMM_W4A4_ENOMEM: return "scratch allocation failed";
    case GEMM_W4A4_ESCRATCH: return "needs more scratch than the no-allocation entry point holds";
    default: return "unknown error";
  }
}

extern "C" int gemm_w4a4(const uint8_t* act, const uint8_t* ascales, const uint8_t* wgt,
                         const uint8_t* wscales, const float* wcscale, const float* bias,
                         const uint16_t* lora_act_in, const uint16_t* lora_up, uint16_t* out,
                         int M, int N, int K, int R, void* stream) {
  return nv_run(-1, false, CallArgs{act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                                    M, N, K, R, stream});
}

extern "C" int gemm_w4a4_f16(const uint8_t* act, const uint8_t* ascales, const uint8_t* wgt,
                             const uint8_t* wscales, const float* wcscale, const float* bias,
                             const uint16_t* lora_act_in, const uint16_t* lora_up, uint16_t* out,
                             int M, int N, int K, int R, void* stream) {
  return nv_run(-1, true, CallArgs{act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                                   M, N, K, R, stream});
}
