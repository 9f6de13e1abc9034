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
constexpr int kLutBytes = 256 * 4;  // E4M3 byte -> packed (s, s) fp16 pair

// BM x BN output tile per workgroup, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) block of 32x32 MFMA tiles. Every pipeline stage covers
// BK = 128 values of k, i.e. 8 NVFP4 scale blocks and 8 MFMA k-steps of 16.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int OCC_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int STAGES = STAGES_;        // LDS ring depth (operand stages)
  static constexpr int OCC = OCC_;              // workgroups per CU the variant is built for
  static constexpr int BK = 128;
  static constexpr int THREADS = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  static constexpr int MI = TM / 32, NI = TN / 32;   // 32x32 MFMA tiles per wave
  static constexpr int ROW_BYTES = BK / 2;      // packed bytes of one row per stage
  static constexpr int CHUNKS = ROW_BYTES / 16; // 16-byte chunks per row per stage
  static constexpr int KSTEPS = BK / 16;        // MFMA k-steps per stage
  static constexpr int QS = BK / 32;            // scale blocks one lane touches per stage
  static constexpr int A_BYTES = BM * ROW_BYTES;
  static constexpr int B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int RING_OFF = 0;
  static constexpr int LUT_OFF = STAGES * STAGE_BYTES;
  static constexpr int LDS_BYTES = LUT_OFF + kLutBytes;
  static constexpr int A_LOADS = BM * CHUNKS / THREADS;  // 16-B chunks per thread per stage
  static constexpr int B_LOADS = BN * CHUNKS / THREADS;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
  static_assert(CHUNKS == 4, "swizzle assumes four 16-byte chunks per row per stage");
  static_assert((BM * CHUNKS) % THREADS == 0 && (BN * CHUNKS) % THREADS == 0,
                "every thread loads the same number of chunks");
  static_assert(THREADS >= 256, "the E4M3 table is filled by the first 256 threads");
  static_assert(LDS_BYTES <= kLdsLimit, "LDS budget exceeded");
  static_assert(LDS_BYTES * OCC <= kLdsLimit, "occupancy target exceeds the LDS budget");
};

// The compiled instances, in variant order. The solver picks among them.
using Cfg256x192 = TileCfg<256, 192, 2, 2, 2, 1>;
using Cfg128x128 = TileCfg<128, 128, 2, 2, 2, 2>;

}  // namespace w4a4
