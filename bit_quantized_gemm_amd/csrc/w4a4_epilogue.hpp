// w4a4_epilogue.hpp — the fused epilogue shared by the NVFP4 and MXFP4 kernels:
// acc * wcscale[n] + bias[n] (the SVDQuant W4A4 on Blackwell page, section
// 6.6), then the rank-R LoRA-up product (section 2's formula adds it after the
// wcscale product; section 6.3 runs it on the same accumulators) as further
// 32x32 MFMA k-steps, then the 16-bit store. Both kernels hold their
// accumulators in the same layout: acc[j][i] is the 32x32 tile of output
// rows m = 32i + l32 (one per lane) and columns n = 32j + 8q + 4g + t in
// element 4q + t, for wave (wm, wn) of the workgroup's BM x BN tile.
#pragma once

#include "w4a4_common.hpp"

namespace w4a4 {

// LoRA chunk size (ranks) and the lora_up transpose task of a thread: 4 ranks
// x 8 columns, ranks fastest across threads.
constexpr int kLoraChunk = 32;
__device__ __forceinline__ int lu_task_r4(int tid) { return (tid % (kLoraChunk / 4)) * 4; }
__device__ __forceinline__ int lu_task_n8(int tid) { return (tid / (kLoraChunk / 4)) * 8; }

// Registers the kernel holds through its K-loop for the epilogue: the first
// LoRA chunk's lora_up pieces, where the side region has no room for them.
struct EpiRegs {
  u32x4 lu[4];
};

// The fast flavour with a side region (C::Side::ON): at the start of the
// kernel, before its first ring DMA, bring wcscale / bias of the tile's
// columns and the first 32 LoRA ranks (act rows; lora_up rows where
// C::Side::LU_ON) into the side region by DMA. These ops are older than every
// ring DMA, so the K-loop's waits for its first stage cover them and the
// epilogue finds them in LDS. Reads past an edge are clamped to valid
// addresses: columns past N and rows past M only reach discarded outputs;
// ranks past R are zeroed by the epilogue.
template <class C, bool GENERAL>
__device__ __forceinline__ void epilogue_prefetch(const Params& p, uint8_t* smem, const int tid,
                                                  const int m0, const int n0, EpiRegs& regs) {
  using S = typename C::Side;
  // each piece's DMA footprint is exactly the bytes the budget solver counted
  static_assert(S::WB_SLOTS / C::THREADS * C::THREADS * 4 == S::WB_BYTES, "WB footprint");
  static_assert(C::BM * 4 / C::THREADS * C::THREADS * 16 == S::LA_BYTES, "LA footprint");
  static_assert(32 * (C::BN / 8) / C::THREADS * C::THREADS * 16 == S::LU_BYTES, "LU footprint");
  if constexpr (!GENERAL && S::ON) {
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = p.N, R = p.R;
#pragma unroll
    for (int u = 0; u < S::WB_SLOTS / C::THREADS; ++u) {
      const int q = u * C::THREADS + tid;          // [2][BN] fp32; slots past 2*BN pad
      const int arr = q < 2 * C::BN ? q / C::BN : 0;
      const int col = q < 2 * C::BN ? q % C::BN : 0;
      const float* src = (arr ? p.bias : p.wcscale) + min(n0 + col, N - 1);
      dma<4>(src, smem + S::WB_OFF + (u * C::THREADS + wave_u * 64) * 4);
    }
    if (R > 0) {
      // LA: slot q = (row, chunk position c) holds data piece c ^ swz(row),
      // ranks 8 (c ^ swz(row)) .. +7 (R % 8 == 0: all in range or all past R)
#pragma unroll
      for (int u = 0; u < C::BM * 4 / C::THREADS; ++u) {
        const int q = u * C::THREADS + tid;
        const int row = q >> 2, dp = (q & 3) ^ swz(row);
        const uint16_t* src = p.lora_act_in + uint32_t(min(m0 + row, p.M - 1)) * uint32_t(R) +
                              uint32_t(min(8 * dp, R - 8));
        dma<16>(src, smem + S::LA_OFF + (u * C::THREADS + wave_u * 64) * 16);
      }
      if constexpr (S::LU_ON) {
        // LU: [32][BN] as stored; rows past R re-read row R-1 (zeroed later)
        constexpr int PER_ROW = C::BN / 8;
#pragma unroll
        for (int u = 0; u < 32 * PER_ROW / C::THREADS; ++u) {
          const int q = u * C::THREADS + tid;
          const int r = q / PER_ROW, c8 = q % PER_ROW;
          const uint16_t* src = p.lora_up + uint32_t(min(r, R - 1)) * uint32_t(N) +
                                uint32_t(min(n0 + 8 * c8, N - 8));
          dma<16>(src, smem + S::LU_OFF + (u * C::THREADS + wave_u * 64) * 16);
        }
      } else if (tid < (kLoraChunk / 4) * (C::BN / 8)) {
        // LU into registers (this thread's transpose task), as the epilogue
        // would load it
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t* src = p.lora_up + uint32_t(min(lu_task_r4(tid) + e, R - 1)) * uint32_t(N);
          regs.lu[e] = *reinterpret_cast<const u32x4*>(src + min(n0 + lu_task_n8(tid), N - 8));
        }
      }
    }
  }
}

// GENERAL: LoRA operands element by element (any R, N, alignment) rather than
// in 16-byte pieces; F16: LoRA operands and output in binary16, else bfloat16.
// The LDS ring (C::RING_BYTES) is dead when this runs and is reused; the side
// region, if any, holds what epilogue_prefetch brought in.
// PART: the launch is one K slice (blockIdx.y) of the tile: its sums times
// wcscale, plus its share of the LoRA term's rank chunks (slice 0 also adds
// bias), are stored in float32 to p.part instead of the output; a reduction
// adds the slices.
template <class C, bool GENERAL, bool F16, bool PART = false>
__device__ __forceinline__ void epilogue(f32x16 (&acc)[C::NI][C::MI], const Params& p, uint8_t* smem,
                                         const int tid, const int m0, const int n0,
                                         const EpiRegs& regs) {
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int M = p.M, N = p.N, R = p.R;
  const bool first = !PART || blockIdx.y == 0;   // the slice that adds bias

  // ---------------- epilogue: *wcscale + bias, + LoRA (same accumulators), bf16 store
  // The first of this lane's four consecutive output columns in (tile j, group q).
  const int ncol0 = n0 + wn * C::TN + 4 * g;          // + 32j + 8q
  const bool n_inside = n0 + C::BN <= N;

  // ---- LoRA-up operands are staged through LDS (the ring is free once the
  // K-loop is done) in chunks of RC ranks = two MFMA k-steps:
  //   LA  lora_act_in rows m0.., [BM][RC] bf16, row-major
  //   LU  lora_up columns n0.., transposed to [BN][RC] bf16
  // so each MFMA operand (8 consecutive ranks of one row) is one 16-byte LDS
  // read. Rows are LR_STRIDE bytes apart (16 bytes of padding), which puts the
  // 16-byte reads of 16 consecutive rows on distinct banks. Ranks past R (and
  // rows past M, columns past N, read clamped) are stored as zero / clamped
  // copies: zero ranks add nothing, clamped rows only reach discarded outputs.
  // With a side region (PRE) LA lives there instead, 64-byte rows with the
  // operand tiles' chunk swizzle (the layout its DMA writes), and LU moves to
  // the start of the ring.
  using S = typename C::Side;
  constexpr bool PRE = !GENERAL && S::ON;
  constexpr int RC = kLoraChunk;
  constexpr int LR_STRIDE = RC * 2 + 16;
  constexpr int LA_OFF = PRE ? S::LA_OFF : 0, LU_OFF = PRE ? 0 : C::BM * LR_STRIDE;
  static_assert(LU_OFF + C::BN * LR_STRIDE <= C::RING_BYTES, "LoRA chunk must fit in the ring");
  // LA: one 16-byte piece = 8 ranks of one row; pieces q = u*THREADS + tid
  constexpr int LA_PIECES = C::BM * RC / 8;
  constexpr int LA_PER = (LA_PIECES + C::THREADS - 1) / C::THREADS;
  // LU: one task = 4 ranks x 8 columns (four 16-byte row pieces), written back
  // as eight 8-byte column pieces; ranks vary fastest across lanes so that 8
  // neighbouring lanes fill one 64-byte LDS row
  constexpr int LU_TASKS = (RC / 4) * (C::BN / 8);
  static_assert(LU_TASKS <= C::THREADS, "one LoRA-up task per thread");
  const bool lu_task = tid < LU_TASKS;
  const int lu_r4 = lu_task_r4(tid);
  const int lu_n8 = lu_task_n8(tid);
  u32x4 la_reg[LA_PER], lu_reg[4];

  auto la_load = [&](int rc0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LA_PER; ++u) {
      const int q = min(u * C::THREADS + tid, LA_PIECES - 1);
      const int row = min(m0 + q / (RC / 8), M - 1);
      const int r = rc0 + (q % (RC / 8)) * 8;
      const uint16_t* src = p.lora_act_in + uint32_t(row) * uint32_t(R);
      if constexpr (!GENERAL) {
        // R % 8 == 0 and r % 8 == 0: the eight ranks are all in range or all
        // out; out-of-range pieces are zeroed when stored
        la_reg[u] = *reinterpret_cast<const u32x4*>(src + min(r, R - 8));
      } else {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint16_t x0 = src[min(r + 2 * t, R - 1)], x1 = src[min(r + 2 * t + 1, R - 1)];
          w[t] = bf16_pair(r + 2 * t < R ? x0 : uint16_t(0), r + 2 * t + 1 < R ? x1 : uint16_t(0));
        }
        la_reg[u] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };
  auto lu_load = [&](int rc0) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rc0 + lu_r4 + e;
      const uint16_t* src = p.lora_up + uint32_t(min(r, R - 1)) * uint32_t(N);
      if constexpr (!GENERAL) {
        // N % 8 == 0: the eight columns are all inside N or all past it; a
        // piece past N re-reads the last one and feeds only discarded outputs
        lu_reg[e] = *reinterpret_cast<const u32x4*>(src + min(n0 + lu_n8, N - 8));
      } else {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint16_t x0 = src[min(n0 + lu_n8 + 2 * t, N - 1)];
          const uint16_t x1 = src[min(n0 + lu_n8 + 2 * t + 1, N - 1)];
          w[t] = r < R ? bf16_pair(x0, x1) : 0u;
        }
        lu_reg[e] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };
  // The fast flavour zeroes ranks past R here rather than at the load, so a
  // prefetch stays in flight until its chunk is stored. With PRE, chunk 0's
  // LA is already in place (only its pieces past R get zeroed), and its LU
  // comes from the side region when it is there.
  auto lora_store = [&](int rc0) __attribute__((always_inline)) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < LA_PER; ++u) {
      const int q = u * C::THREADS + tid;
      const int row = q / (RC / 8), dp = q % (RC / 8);
      const bool keep = GENERAL || rc0 + dp * 8 < R;
      if constexpr (PRE) {
        // The swizzle pairs chunk position x of a row with data piece
        // x ^ swz(row). Chunk 0: this thread's DMA filled position dp with
        // piece dp ^ swz(row); zero it if those ranks are past R. Later
        // chunks: la_reg[u] holds piece dp, which goes to position dp ^ swz(row).
        const int dx = dp ^ swz(row);
        if (rc0 == 0) {
          if (dx * 8 >= R) *reinterpret_cast<u32x4*>(smem + LA_OFF + row * 64 + dp * 16) = zero;
        } else {
          *reinterpret_cast<u32x4*>(smem + LA_OFF + row * 64 + dx * 16) = keep ? la_reg[u] : zero;
        }
      } else if (LA_PIECES % C::THREADS == 0 || q < LA_PIECES) {
        *reinterpret_cast<u32x4*>(smem + LA_OFF + row * LR_STRIDE + dp * 16) = keep ? la_reg[u] : zero;
      }
    }
    if constexpr (PRE && S::LU_ON) {
      if (rc0 == 0 && lu_task) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lu_reg[e] = *reinterpret_cast<const u32x4*>(smem + S::LU_OFF + ((lu_r4 + e) * C::BN + lu_n8) * 2);
      }
    } else if constexpr (PRE) {
      if (rc0 == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lu_reg[e] = regs.lu[e];
      }
    }
    if constexpr (!GENERAL) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (rc0 + lu_r4 + e >= R) lu_reg[e] = zero;
    }
    if (lu_task) {
      // column c of the four row pieces -> LU[n8 + c][r4 .. r4+3]
      uint8_t* dst = smem + LU_OFF + lu_n8 * LR_STRIDE + lu_r4 * 2;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const u32x2 lo = {__builtin_amdgcn_perm(lu_reg[1][h], lu_reg[0][h], 0x05040100u),
                          __builtin_amdgcn_perm(lu_reg[3][h], lu_reg[2][h], 0x05040100u)};
        const u32x2 hi = {__builtin_amdgcn_perm(lu_reg[1][h], lu_reg[0][h], 0x07060302u),
                          __builtin_amdgcn_perm(lu_reg[3][h], lu_reg[2][h], 0x07060302u)};
        *reinterpret_cast<u32x2*>(dst + (2 * h) * LR_STRIDE) = lo;
        *reinterpret_cast<u32x2*>(dst + (2 * h + 1) * LR_STRIDE) = hi;
      }
    }
  };

  // K slices share the LoRA term: slice s takes rank chunks s, s + S, ...
  // (the term is a sum over chunks), so no slice waits on all of them.
  const int nchunks = (R + RC - 1) / RC;
  const int c0 = PART ? int(blockIdx.y) : 0, cstep = PART ? int(gridDim.y) : 1;
  if (c0 < nchunks) {
    if (!PRE || c0 != 0) {
      la_load(c0 * RC);
      lu_load(c0 * RC);
    }
  }

  // Per-column factor at columns ncol0 + 32j + 8q + (0..3), clamped at the N
  // edge. n is a multiple of 4, so one 16-byte read serves the four columns
  // when both vectors are 16-byte aligned; the interface only promises 4 bytes.
  const bool wb16 = ((reinterpret_cast<uintptr_t>(p.wcscale) | reinterpret_cast<uintptr_t>(p.bias)) & 15u) == 0;
  auto col4 = [&](const float* v, int j, int q) __attribute__((always_inline)) {
    const int n = ncol0 + 32 * j + 8 * q;
    if (n_inside && wb16) return *reinterpret_cast<const f32x4*>(v + n);
    return f32x4{v[min(n, N - 1)], v[min(n + 1, N - 1)], v[min(n + 2, N - 1)], v[min(n + 3, N - 1)]};
  };

  // S * wcscale[n] + bias[n] (the LoRA terms are added on top by the MFMAs
  // below); with PRE the factors come from the side region
  const uint32_t wb_rd = S::WB_OFF + (wn * C::TN + 4 * g) * 4;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 w, b;
      if constexpr (PRE) {
        w = *reinterpret_cast<const f32x4*>(smem + wb_rd + (32 * j + 8 * q) * 4);
        b = *reinterpret_cast<const f32x4*>(smem + wb_rd + (C::BN + 32 * j + 8 * q) * 4);
      } else {
        w = col4(p.wcscale, j, q);
        b = col4(p.bias, j, q);
      }
      if (!first) b = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[j][i][4 * q + t] = __builtin_fmaf(acc[j][i][4 * q + t], w[t], b[t]);
    }
  }

  // LoRA-up: per chunk, store the staged operands, prefetch the next chunk,
  // then two k-steps of v_mfma_f32_32x32x16_bf16 (same accumulator layout as
  // the K-loop: lora_up as the A operand, rows n; lora_act_in as B, rows m).
  // Lane (l32, g) feeds ranks 8g .. 8g+7 of each 16-rank k-step.
  const int la_row = wm * C::TM + l32;   // + 32i: the same swizzle
  const uint32_t la_rd = PRE ? LA_OFF + la_row * 64 : LA_OFF + la_row * LR_STRIDE + g * 16;
  const uint32_t lu_rd = LU_OFF + (wn * C::TN + l32) * LR_STRIDE + g * 16;
  for (int c = c0; c < nchunks; c += cstep) {
    wait_vm_lgkm0<0>();
    wg_barrier();   // every wave is done with the ring / the previous chunk
    lora_store(c * RC);
    if (c + cstep < nchunks) {
      la_load((c + cstep) * RC);
      lu_load((c + cstep) * RC);
    }
    wait_vm_lgkm0<63>();
    wg_barrier();
#pragma unroll
    for (int s = 0; s < RC / 16; ++s) {
      if (s > 0 && c * RC + 16 * s >= R) break;   // an all-zero k-step
      u32x4 la[C::MI], lu[C::NI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        if constexpr (PRE)
          la[i] = *reinterpret_cast<const u32x4*>(smem + la_rd + i * 32 * 64 + (((2 * s + g) ^ swz(la_row)) << 4));
        else
          la[i] = *reinterpret_cast<const u32x4*>(smem + la_rd + i * 32 * LR_STRIDE + s * 32);
      }
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
        lu[j] = *reinterpret_cast<const u32x4*>(smem + lu_rd + j * 32 * LR_STRIDE + s * 32);
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int i = 0; i < C::MI; ++i) acc[j][i] = lora_mfma<F16>(lu[j], la[i], acc[j][i]);
    }
  }

  if constexpr (PART) {
    // float32 sums of this slice, staged through LDS as whole rows, then
    // stored as 16-byte pieces of rows of p.part (N % 4 == 0, 16-byte aligned)
    wait_vm_lgkm0<0>();
    wg_barrier();
    constexpr int F_STRIDE = C::BN * 4 + 16;
    static_assert(C::BM * F_STRIDE <= C::RING_BYTES, "float32 tile must fit in the ring");
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
          const int ml = wm * C::TM + 32 * i + l32;
          const int nl = wn * C::TN + 32 * j + 8 * q + 4 * g;
          *reinterpret_cast<f32x4*>(smem + ml * F_STRIDE + nl * 4) =
              f32x4{acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
        }
    wait_vm_lgkm0<63>();
    wg_barrier();
    constexpr int F_PER_ROW = C::BN / 4;
    constexpr int F_PIECES = C::BM * F_PER_ROW;
    static_assert(F_PIECES % C::THREADS == 0, "whole store rounds");
    float* const dst = p.part + size_t(blockIdx.y) * size_t(p.part_rows) * size_t(N);
#pragma unroll
    for (int u = 0; u < F_PIECES / C::THREADS; ++u) {
      const int piece = u * C::THREADS + tid;
      const int rl = piece / F_PER_ROW, cl = (piece % F_PER_ROW) * 4;
      const int row = m0 + rl, col = n0 + cl;
      if (row >= M || col >= N) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(smem + rl * F_STRIDE + cl * 4);
      *reinterpret_cast<f32x4*>(dst + size_t(row - p.part_row0) * size_t(N) + size_t(col)) = v;
    }
    return;
  }

  // bf16 (round to nearest even), staged through LDS: the tile is row-major
  // with a padded row stride (OUT_STRIDE bytes) so the 8-byte writes of 32
  // rows at once spread over the banks. The barrier makes sure every wave is
  // done with the ring (K-loop) and with the LoRA operands.
  wait_vm_lgkm0<0>();
  wg_barrier();
  constexpr int OUT_STRIDE = C::BN * 2 + 16;
  static_assert(C::BM * OUT_STRIDE <= C::RING_BYTES, "output tile must fit in the ring");
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int ml = wm * C::TM + 32 * i + l32;
        const int nl = wn * C::TN + 32 * j + 8 * q + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        if constexpr (F16) {
          const f16x4 v = {_Float16(acc[j][i][4 * q]), _Float16(acc[j][i][4 * q + 1]),
                           _Float16(acc[j][i][4 * q + 2]), _Float16(acc[j][i][4 * q + 3])};
          *reinterpret_cast<f16x4*>(smem + ml * OUT_STRIDE + nl * 2) = v;
        } else {
          const bf16x4 v = {__bf16(acc[j][i][4 * q]), __bf16(acc[j][i][4 * q + 1]),
                            __bf16(acc[j][i][4 * q + 2]), __bf16(acc[j][i][4 * q + 3])};
          *reinterpret_cast<bf16x4*>(smem + ml * OUT_STRIDE + nl * 2) = v;
        }
      }
    }
  }
  wait_vm_lgkm0<63>();
  wg_barrier();

  // LDS -> HBM in 16-byte pieces of whole output rows (8 columns each), as
  // non-temporal stores: the output is not read again by this launch, and
  // keeping it out of the way of the operands in L2 measured 1-2 % faster.
  constexpr int PIECES_PER_ROW = C::BN / 8;
  constexpr int PIECES = C::BM * PIECES_PER_ROW;
  static_assert(PIECES % C::THREADS == 0, "whole store rounds");
  // A piece wholly inside N is one 16-byte store whenever output rows are
  // 16-byte aligned (N % 8 == 0, aligned out), also in a tile at the N edge;
  // element stores only otherwise, and never past N.
  const bool vec_ok = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15u) == 0;
  if (vec_ok && n_inside) {
    // the common case, kept free of per-piece column checks
#pragma unroll
    for (int u = 0; u < PIECES / C::THREADS; ++u) {
      const int piece = u * C::THREADS + tid;
      const int rl = piece / PIECES_PER_ROW, cl = (piece % PIECES_PER_ROW) * 8;
      const int row = m0 + rl;
      if (row >= M) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + rl * OUT_STRIDE + cl * 2);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.out + uint32_t(row) * uint32_t(N) + uint32_t(n0 + cl)));
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < PIECES / C::THREADS; ++u) {
    const int piece = u * C::THREADS + tid;
    const int rl = piece / PIECES_PER_ROW, cl = (piece % PIECES_PER_ROW) * 8;
    const int row = m0 + rl;
    const int left = N - (n0 + cl);   // columns of this piece inside N
    if (row >= M || left <= 0) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + rl * OUT_STRIDE + cl * 2);
    uint16_t* dst = p.out + uint32_t(row) * uint32_t(N) + uint32_t(n0 + cl);
    if (vec_ok && left >= 8) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < left) dst[e] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// The slices of a K-sliced launch added: part holds S planes of rows x N
// float32 sums (slice 0 carries bias and the LoRA term), summed in slice
// order and rounded to the output type (nearest even) into output rows
// row0 .. row0 + rows - 1. One thread per four consecutive outputs
// (N % 4 == 0, out 8-byte aligned).
template <bool F16>
__global__ __launch_bounds__(256) void split_k_reduce(const float* part, uint16_t* out, int rows, int N, int S,
                                                      int row0) {
  const uint32_t q = blockIdx.x * 256u + threadIdx.x;
  if (q >= uint32_t(rows) * uint32_t(N >> 2)) return;
  const size_t plane = size_t(rows) * size_t(N);
  f32x4 v = *reinterpret_cast<const f32x4*>(part + size_t(q) * 4);
  for (int k = 1; k < S; ++k) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(part + size_t(k) * plane + size_t(q) * 4);
    v = f32x4{v[0] + w[0], v[1] + w[1], v[2] + w[2], v[3] + w[3]};
  }
  uint16_t* dst = out + size_t(row0) * size_t(N) + size_t(q) * 4;
  if constexpr (F16) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<f16x4*>(dst) = f16x4{_Float16(v[0]), _Float16(v[1]), _Float16(v[2]), _Float16(v[3])};
  } else {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{__bf16(v[0]), __bf16(v[1]), __bf16(v[2]), __bf16(v[3])};
  }
}

}  // namespace w4a4
