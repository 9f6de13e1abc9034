// w4a4_layout.hpp — compile-time tile shapes and LDS layout of the W4A4 kernels.
//
// One struct, TileCfg, fixes every size the kernel carves out of LDS. The host
// budget solver reads the very same constants, so the bytes it budgets are the
// bytes the kernel uses; a test compares them with the LDS size the compiler
// wrote into each code object. (The SVDQuant W4A4 on Blackwell page, section 7,
// shows how a budget estimate that drifted from the real layout silently
// halved the number of K-blocks in flight; sharing the struct removes that
// drift, and the code-object check catches what remains.)
#pragma once

#include <stdint.h>

namespace w4a4 {

constexpr int kLdsLimit = 163840;   // LDS one workgroup may use on gfx950 (160 KiB)
constexpr int kNumCUs = 256;        // MI355X compute units
constexpr int kWave = 64;           // CDNA wavefront width

// The epilogue's side region, after the ring, where the LDS budget of one
// workgroup (kLdsLimit / OCC) allows it: what the epilogue needs first,
// brought in by DMA at the start of the kernel so that its latency hides
// behind the K-loop.
//   WB  wcscale then bias of the tile's BN columns, fp32 [2][BN], padded to
//       whole rounds of 4-byte DMA pieces
//   LA  LoRA ranks 0..31 of the tile's BM act rows, 16-bit [BM][64 bytes],
//       16-byte chunks XOR-swizzled by row as the operand tiles
//   LU  lora_up rows 0..31 at the tile's BN columns as stored, 16-bit
//       [32][BN] (only where it still fits; the epilogue transposes it)
template <int BM, int BN, int THREADS, int OCC, int RING>
struct EpiSide {
  static constexpr int WB_SLOTS = (2 * BN + THREADS - 1) / THREADS * THREADS;
  static constexpr int WB_BYTES = WB_SLOTS * 4;
  static constexpr int LA_BYTES = BM * 64;
  static constexpr int LU_BYTES = 32 * BN * 2;
  static constexpr int BUDGET = kLdsLimit / OCC;
  static constexpr bool ON = RING + WB_BYTES + LA_BYTES <= BUDGET;
  static constexpr bool LU_ON = ON && RING + WB_BYTES + LA_BYTES + LU_BYTES <= BUDGET;
  static constexpr int WB_OFF = RING;
  static constexpr int LA_OFF = WB_OFF + WB_BYTES;
  static constexpr int LU_OFF = LA_OFF + LA_BYTES;
  static constexpr int BYTES = ON ? WB_BYTES + LA_BYTES + (LU_ON ? LU_BYTES : 0) : 0;
  static_assert(RING % 16 == 0 && WB_BYTES % 16 == 0, "16-byte aligned regions");
  static_assert((BM * 4) % THREADS == 0 && (32 * BN / 8) % THREADS == 0, "whole DMA rounds");
};

// BM x BN output tile per workgroup, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) block of 32x32 MFMA tiles. Every pipeline stage covers
// BK = 128 values of k, i.e. 8 NVFP4 scale blocks and 8 MFMA k-steps of 16.
//
// One LDS ring stage holds, in this order:
//   A  packed act  [BM rows][64 bytes]  16-byte chunks XOR-swizzled by row
//   B  packed wgt  [BN rows][64 bytes]  same swizzle
//   SA act scales  fp16 [4 k-block pairs][BM rows][2]
//   SB wgt scales  fp16 [4 k-block pairs][BN rows][2]
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int OCC_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int STAGES = STAGES_;        // LDS ring depth (stages in flight)
  static constexpr int OCC = OCC_;              // workgroups per CU the variant is built for
  static constexpr int BK = 128;
  static constexpr int THREADS = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  static constexpr int MI = TM / 32, NI = TN / 32;   // 32x32 MFMA tiles per wave
  static constexpr int ROW_BYTES = BK / 2;      // packed bytes of one row per stage
  static constexpr int KBLK = BK / 16;          // scale blocks (= MFMA k-steps) per stage
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = A_OFF + BM * ROW_BYTES;
  static constexpr int SA_OFF = B_OFF + BN * ROW_BYTES;
  static constexpr int SB_OFF = SA_OFF + KBLK * BM * 2;
  static constexpr int STAGE_BYTES = SB_OFF + KBLK * BN * 2;
  static constexpr int PACKED_BYTES = SA_OFF;   // bytes moved by DMA per stage
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  using Side = EpiSide<BM, BN, THREADS, OCC, RING_BYTES>;
  static constexpr int LDS_BYTES = RING_BYTES + Side::BYTES;
  // scale loader: one thread per 8 consecutive rows of one k-block pair
  static constexpr int SA_THREADS = BM / 2;     // (KBLK / 2) * (BM / 8)
  static constexpr int SB_THREADS = BN / 2;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(BK == 128, "the lane <-> k mapping assumes 8 k-steps per stage");
  static_assert(PACKED_BYTES % (THREADS * 16) == 0, "whole 16-byte DMA rounds per stage");
  static_assert(SA_THREADS + SB_THREADS <= THREADS, "one scale chunk per thread");
  static_assert(STAGES == 4, "the pipeline below is written for a 4-deep ring");
  static_assert(LDS_BYTES <= kLdsLimit, "LDS budget exceeded");
  static_assert(LDS_BYTES * OCC <= kLdsLimit, "occupancy target exceeds the LDS budget");
};

// The compiled instances, in variant order. The solver picks among them.
using Cfg256x192 = TileCfg<256, 192, 2, 2, 4, 1>;
using Cfg128x128 = TileCfg<128, 128, 2, 2, 4, 2>;
using Cfg256x128 = TileCfg<256, 128, 2, 2, 4, 1>;

// MXFP4 kernel: BM x BN tile, WM x WN waves of (BM/WM) x (BN/WN), 32x32x64
// scaled FP4 MFMAs. A stage covers BK = 128 values of k = 2 MFMA k-steps = 4
// UE8M0 scale blocks of 32. One ring stage holds, in this order:
//   A  packed act  [BM rows][64 bytes]  16-byte chunks XOR-swizzled by row
//   B  packed wgt  [BN rows][64 bytes]  same swizzle
//   S  raw UE8M0 scale bytes: act [4][BM] then wgt [4][BN] ([k-block][row],
//      the global layout's order), padded to whole 4-byte DMA rounds
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int OCC_>
struct MxTileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int STAGES = STAGES_, OCC = OCC_;
  static constexpr int BK = 128;
  static constexpr int THREADS = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MI = TM / 32, NI = TN / 32;
  static constexpr int ROW_BYTES = BK / 2;
  static constexpr int KBLK = BK / 32;            // scale blocks per stage
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = A_OFF + BM * ROW_BYTES;
  static constexpr int SA_OFF = B_OFF + BN * ROW_BYTES;
  static constexpr int SB_OFF = SA_OFF + KBLK * BM;
  static constexpr int SCALE_BYTES = KBLK * (BM + BN);
  static constexpr int SCALE_ROUNDS = (SCALE_BYTES + THREADS * 4 - 1) / (THREADS * 4);
  static constexpr int PACKED_BYTES = SA_OFF;
  static constexpr int STAGE_BYTES = SA_OFF + SCALE_ROUNDS * THREADS * 4;
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  using Side = EpiSide<BM, BN, THREADS, OCC, RING_BYTES>;
  static constexpr int LDS_BYTES = RING_BYTES + Side::BYTES;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(BM % 4 == 0 && BN % 4 == 0, "4-row scale DMA pieces");
  static_assert(PACKED_BYTES % (THREADS * 16) == 0 && B_OFF % (THREADS * 16) == 0,
                "whole 16-byte DMA rounds per operand");
  static_assert(STAGES >= 3, "at least two stages in flight");
  static_assert(LDS_BYTES * OCC <= kLdsLimit, "LDS budget exceeded");
};

// 256 x 192, not 256 x 256: 256 accumulators fill the accumulator file and
// the epilogue then spills; 192 leave it room (as in the NVFP4 kernel).
using MxCfg256x192 = MxTileCfg<256, 192, 2, 2, 4, 1>;
using MxCfg128x128 = MxTileCfg<128, 128, 2, 2, 4, 2>;

}  // namespace w4a4
