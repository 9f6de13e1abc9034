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

// ---------------------------------------------------------------- LDS budget solver
//
// A workgroup's LDS share (kLdsLimit / OCC) holds the operand ring — DEPTH
// stages in flight, the K-loop's latency cover — and, beside it where room is
// left, the epilogue's side region: what the epilogue needs first, brought in
// by DMA at the start of the kernel so that its latency hides behind the
// K-loop:
//   WB  wcscale then bias of the tile's BN columns, fp32 [2][BN], padded to
//       whole rounds of 4-byte DMA pieces
//   LA  LoRA ranks 0..31 of the tile's BM act rows, 16-bit [BM][64 bytes],
//       16-byte chunks XOR-swizzled by row as the operand tiles
//   LU  lora_up rows 0..31 at the tile's BN columns as stored, 16-bit [32][BN]
// Later LoRA chunks (ranks 32 and up) never compete with the ring: they are
// staged through the drained ring after the K-loop (aliasing, not a second
// budget line).
//
// The solve: with the side-first policy, the deepest ring (up to MAX_DEPTH)
// that leaves room for the whole side region; failing MIN_DEPTH that way, WB
// and LA only; failing that, no side region. With the depth-first policy, the
// deepest ring first, then whichever side pieces still fit. Each count is the
// footprint its writer has (the epilogue static_asserts its DMA pieces against
// these constants), so a miscounted buffer shows up as a compile error or as a
// mismatch with the LDS size the compiler writes into the code object, instead
// of as a silently shallower ring — the failure the SVDQuant W4A4 on Blackwell
// page (section 7) traced to a LoRA-up buffer counted twice.
enum : int { kPlaceRing = 0, kPlaceSideAct = 1, kPlaceSideActUp = 2 };   // first LoRA chunk
enum : int { kDepthFirst = 0, kSideFirst = 1 };                          // solver policy
constexpr int kMinDepth = 3;    // the K-loop's schedule needs stage st+1 in flight while st computes
constexpr int kMaxDepth = 4;    // deeper rings measured slower (MXFP4: 5 stages 2-4 % slower than 4)

// The LoRA-up side piece is multiplied by this factor in the budget: 1 is the
// true count. A test builds the header with 2 to show what a double count does.
#ifndef W4A4_LU_ACCOUNTING_FACTOR
#define W4A4_LU_ACCOUNTING_FACTOR 1
#endif

struct Budget {
  int depth;        // ring stages
  int place;        // where the first LoRA chunk lives (kPlace*)
  int wb_bytes, la_bytes, lu_bytes;   // side-region pieces present (0 when absent)
  int ring_bytes, side_bytes, lds_bytes;
};

constexpr Budget make_budget(int depth, int place, int stage, int wb, int la, int lu) {
  const int w = place >= kPlaceSideAct ? wb : 0, a = place >= kPlaceSideAct ? la : 0;
  const int u = place == kPlaceSideActUp ? lu : 0;
  return Budget{depth, place, w, a, u, depth * stage, w + a + u, depth * stage + w + a + u};
}

constexpr Budget solve_budget(int stage, int wb, int la, int lu, int share, int policy,
                              int min_depth = kMinDepth, int max_depth = kMaxDepth) {
  const int fit = share / stage;                          // deepest ring alone
  if (fit < min_depth) return make_budget(0, kPlaceRing, stage, wb, la, lu);   // does not fit
  if (policy == kSideFirst) {
    const int full = (share - wb - la - lu) / stage;
    if (share >= wb + la + lu && full >= min_depth)
      return make_budget(full < max_depth ? full : max_depth, kPlaceSideActUp, stage, wb, la, lu);
    const int part = (share - wb - la) / stage;
    if (share >= wb + la && part >= min_depth)
      return make_budget(part < max_depth ? part : max_depth, kPlaceSideAct, stage, wb, la, lu);
    return make_budget(fit < max_depth ? fit : max_depth, kPlaceRing, stage, wb, la, lu);
  }
  const int d = fit < max_depth ? fit : max_depth;
  const int left = share - d * stage;
  const int place = left >= wb + la + lu ? kPlaceSideActUp : left >= wb + la ? kPlaceSideAct : kPlaceRing;
  return make_budget(d, place, stage, wb, la, lu);
}

// Side-region piece sizes of a BM x BN tile run by THREADS threads.
template <int BM, int BN, int THREADS>
struct SidePieces {
  static constexpr int WB_SLOTS = (2 * BN + THREADS - 1) / THREADS * THREADS;
  static constexpr int WB = WB_SLOTS * 4;
  static constexpr int LA = BM * 64;
  static constexpr int LU = 32 * BN * 2;
};

// The side region as the kernels carve it, from a solved budget.
template <int BM, int BN, int THREADS, int RING, int PLACE>
struct EpiSide {
  using P = SidePieces<BM, BN, THREADS>;
  static constexpr int WB_SLOTS = P::WB_SLOTS;
  static constexpr int WB_BYTES = P::WB;
  static constexpr int LA_BYTES = P::LA;
  static constexpr int LU_BYTES = P::LU;
  static constexpr bool ON = PLACE >= kPlaceSideAct;
  static constexpr bool LU_ON = PLACE == kPlaceSideActUp;
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
// With KG = 2 k-groups, each wave block is computed by two waves, one taking
// k-steps 0-3 of every stage and the other k-steps 4-7, whose partial sums
// meet in LDS after the K-loop (a tile with few rows then still occupies
// every SIMD with a wave tile big enough to keep the decode per MFMA low).
// OCC workgroups share a compute unit; POLICY steers the budget solve, which
// sets the ring depth (STAGES) and the side region.
//
// One LDS ring stage holds, in this order:
//   A  packed act  [BM rows][64 bytes]  16-byte chunks XOR-swizzled by row
//   B  packed wgt  [BN rows][64 bytes]  same swizzle
//   SA act scales  fp16 [4 k-block pairs][BM rows][2]
//   SB wgt scales  fp16 [4 k-block pairs][BN rows][2]
// The geometry of a tile (what one ring stage holds), apart from its budget.
template <int BM_, int BN_, int WM_, int WN_, int KG_ = 1>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, KG = KG_;
  static constexpr int BK = 128;
  static constexpr int THREADS = WM * WN * KG * kWave;
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
  using Pieces = SidePieces<BM, BN, THREADS>;
  static_assert(KG == 1 || (KG == 2 && MI % 2 == 0), "k-groups split the 8 k-steps and the m-tiles in two");
};

template <int BM_, int BN_, int WM_, int WN_, int OCC_, int POLICY_, int KG_ = 1>
struct TileCfg : TileShape<BM_, BN_, WM_, WN_, KG_> {
  using G = TileShape<BM_, BN_, WM_, WN_, KG_>;
  using G::BM, G::BN, G::THREADS, G::TM, G::TN, G::BK, G::STAGE_BYTES, G::PACKED_BYTES;
  static constexpr int OCC = OCC_;              // workgroups per CU the variant is built for
  static constexpr int POLICY = POLICY_;
  static constexpr Budget BUDGET = solve_budget(STAGE_BYTES, G::Pieces::WB, G::Pieces::LA,
                                                G::Pieces::LU * W4A4_LU_ACCOUNTING_FACTOR,
                                                kLdsLimit / OCC, POLICY);
  static constexpr int STAGES = BUDGET.depth;   // LDS ring depth (stages in flight)
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  using Side = EpiSide<BM, BN, THREADS, RING_BYTES, BUDGET.place>;
  static constexpr int LDS_BYTES = RING_BYTES + Side::BYTES;
  // scale loader: one thread per 8 consecutive rows of one k-block pair
  static constexpr int SA_THREADS = BM / 2;     // (KBLK / 2) * (BM / 8)
  static constexpr int SB_THREADS = BN / 2;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(BK == 128, "the lane <-> k mapping assumes 8 k-steps per stage");
  static_assert(PACKED_BYTES % (THREADS * 16) == 0, "whole 16-byte DMA rounds per stage");
  static_assert(SA_THREADS + SB_THREADS <= THREADS, "one scale chunk per thread");
  static_assert(STAGES >= kMinDepth, "the ring does not fit the LDS share");
  static_assert(LDS_BYTES == BUDGET.lds_bytes, "the carved layout is the solved budget");
  static_assert(LDS_BYTES * OCC <= kLdsLimit, "occupancy target exceeds the LDS budget");
};

// The tile as the epilogue sees it once the k-groups have exchanged partial
// sums: k-group kg of wave row wm keeps m-tiles [kg MI/KG, (kg+1) MI/KG) of
// that row's wave tile, i.e. it is wave row wm*KG + kg of a KG-times finer
// grid of waves (same LDS layout, same threads).
template <class C>
struct EpiView : C {
  static constexpr int WM = C::WM * C::KG, TM = C::TM / C::KG, MI = C::MI / C::KG;
};

// The compiled instances, in variant order. The solver picks among them.
using Cfg256x192 = TileCfg<256, 192, 2, 2, 1, kDepthFirst>;   // ring 4, side WB+LA
using Cfg128x128 = TileCfg<128, 128, 2, 2, 2, kDepthFirst>;   // ring 4, no side region
using Cfg256x128 = TileCfg<256, 128, 2, 2, 1, kDepthFirst>;   // ring 4, side WB+LA+LU
using Cfg128x128S = TileCfg<128, 128, 2, 2, 2, kSideFirst>;   // ring 3, side WB+LA+LU
using Cfg64x192K = TileCfg<64, 192, 1, 2, 1, kDepthFirst, 2>; // ring 4, side WB+LA+LU; 2 k-groups

// MXFP4 kernel: BM x BN tile, WM x WN waves of (BM/WM) x (BN/WN), 32x32x64
// scaled FP4 MFMAs. A stage covers BK = 128 values of k = 2 MFMA k-steps = 4
// UE8M0 scale blocks of 32. One ring stage holds, in this order:
//   A  packed act  [BM rows][64 bytes]  16-byte chunks XOR-swizzled by row
//   B  packed wgt  [BN rows][64 bytes]  same swizzle
//   S  raw UE8M0 scale bytes: act [4][BM] then wgt [4][BN] ([k-block][row],
//      the global layout's order), padded to whole 4-byte DMA rounds
template <int BM_, int BN_, int WM_, int WN_>
struct MxTileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, KG = 1;
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
  using Pieces = SidePieces<BM, BN, THREADS>;
};

template <int BM_, int BN_, int WM_, int WN_, int OCC_, int POLICY_>
struct MxTileCfg : MxTileShape<BM_, BN_, WM_, WN_> {
  using G = MxTileShape<BM_, BN_, WM_, WN_>;
  using G::BM, G::BN, G::THREADS, G::TM, G::TN, G::B_OFF, G::STAGE_BYTES, G::PACKED_BYTES;
  static constexpr int OCC = OCC_, POLICY = POLICY_;
  static constexpr Budget BUDGET = solve_budget(STAGE_BYTES, G::Pieces::WB, G::Pieces::LA,
                                                G::Pieces::LU * W4A4_LU_ACCOUNTING_FACTOR,
                                                kLdsLimit / OCC, POLICY);
  static constexpr int STAGES = BUDGET.depth;
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  using Side = EpiSide<BM, BN, THREADS, RING_BYTES, BUDGET.place>;
  static constexpr int LDS_BYTES = RING_BYTES + Side::BYTES;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(BM % 4 == 0 && BN % 4 == 0, "4-row scale DMA pieces");
  static_assert(PACKED_BYTES % (THREADS * 16) == 0 && B_OFF % (THREADS * 16) == 0,
                "whole 16-byte DMA rounds per operand");
  static_assert(STAGES >= kMinDepth, "the ring does not fit the LDS share");
  static_assert(LDS_BYTES == BUDGET.lds_bytes, "the carved layout is the solved budget");
  static_assert(LDS_BYTES * OCC <= kLdsLimit, "LDS budget exceeded");
};

// 256 x 192, not 256 x 256: 256 accumulators fill the accumulator file and
// the epilogue then spills; 192 leave it room (as in the NVFP4 kernel).
using MxCfg256x192 = MxTileCfg<256, 192, 2, 2, 1, kSideFirst>;   // ring 4, side WB+LA+LU
using MxCfg128x128 = MxTileCfg<128, 128, 2, 2, 2, kDepthFirst>;  // ring 4, side WB+LA

}  // namespace w4a4
