/*
 * w4a4_probes.h — C ABI of libw4a4_probes.so: measurement aids that sit beside
 * the fused W4A4 GEMM library (include/gemm_w4a4.h) but are not part of the
 * operator. They give the figures the operator's performance is compared
 * with: the attainable rate of each matrix instruction under full-chip
 * load, and the two candidate ways of running NVFP4's block-scaled product on
 * gfx950's matrix cores.
 *
 * Return codes are gemm_w4a4.h's. Every pointer is a device pointer owned by
 * the caller; nothing is allocated, nothing synchronised: a successful call
 * only enqueues work on `stream` (a hipStream_t passed as void*, NULL = the
 * null stream).
 */
#ifndef W4A4_PROBES_H
#define W4A4_PROBES_H

#include <stdint.h>

#include "gemm_w4a4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * w4a4_probe_mfma_peak: the
 * attainable rate of one MFMA kind under full-chip load (the third peak the
 * measurement plan asks for beside the published ones). Launches
 * W4A4_PROBE_GROUPS workgroups of four waves; every wave issues iters x 8
 * back-to-back MFMAs into independent accumulators:
 *   kind 0  v_mfma_f32_32x32x16_f16     (the NVFP4 K-loop's; 32768 flop each)
 *   kind 1  v_mfma_scale_f32_32x32x64_f8f6f4, FP4 operands (the MXFP4
 *           K-loop's; 131072 flop each)
 *   kind 2  v_mfma_f32_32x32x16_bf16    (the LoRA k-steps'; 32768 flop each)
 * clocks: caller-owned device buffer of 2 * W4A4_PROBE_GROUPS uint64, 8-byte
 * aligned; workgroup g writes its shader-clock cycles (s_memtime) at [2g] and
 * its 100 MHz wall-clock ticks (s_memrealtime) at [2g+1] over the MFMA loop.
 * Flops per launch = W4A4_PROBE_GROUPS * 4 * iters * 8 * (flop each).
 * Returns GEMM_W4A4_EINVAL (kind not 0..2, iters < 1, clocks NULL),
 * GEMM_W4A4_EALIGN, GEMM_W4A4_EDEVICE, GEMM_W4A4_ELAUNCH or GEMM_W4A4_OK.
 */
#define W4A4_PROBE_GROUPS 256
int w4a4_probe_mfma_peak(int kind, int iters, uint64_t* clocks, void* stream);

/*
 * w4a4_probe_route_core: the
 * per-block arithmetic of the two ways to run NVFP4 (E2M1 codes, one E4M3
 * scale per 16 k; the SVDQuant W4A4 on Blackwell page, section 3.1) on
 * gfx950's matrix cores, for one wave tile of 4 x 3 MFMA tiles of 32x32, on
 * register-resident operands (no memory traffic). Launches
 * W4A4_PROBE_GROUPS workgroups of four waves; every wave runs `blocks`
 * 16-k scale blocks:
 *   route 0  decode to fp16 (4 conversions + 4 packed multiplies per lane,
 *            tile and block) and 12 v_mfma_f32_32x32x16_f16 — the route
 *            gemm_w4a4 takes;
 *   route 1  12 v_mfma_scale_f32_32x32x64_f8f6f4 on the raw FP4 codes, one
 *            16-k block in 16 of the 64 k slots (E8M0 scales 1.0, fresh
 *            partial sums), then acc += partial * (sa * sw) per element.
 * Useful work per launch: W4A4_PROBE_GROUPS * 4 * blocks * 12 * 32768
 * flop (32x32x16 multiply-adds per MFMA), either route. clocks as for
 * w4a4_probe_mfma_peak. Returns GEMM_W4A4_EINVAL (route not 0..1, blocks < 1,
 * clocks NULL), GEMM_W4A4_EALIGN, GEMM_W4A4_EDEVICE, GEMM_W4A4_ELAUNCH or
 * GEMM_W4A4_OK.
 */
int w4a4_probe_route_core(int route, int blocks, uint64_t* clocks, void* stream);

/*
 * w4a4_probe_route_b_tile: one 32 x 32 output tile computed
 * by route 1 above, so that its exactness can be checked.
 *   out[m][n] = sum over k-blocks b of E4M3(ascales[b][m]) * E4M3(wscales[b][n])
 *               * sum over the block's 16 k of E2M1(act[m][k]) * E2M1(wgt[n][k])
 * act, wgt: device, [32][K/2] bytes, two E2M1 codes a byte (low nibble = even
 * k), 4-byte aligned. ascales, wscales: device, [K/16][32] E4M3 bytes. out:
 * device, caller-owned [32][32] float32, 4-byte aligned, fully overwritten.
 * 16 <= K <= W4A4_PROBE_ROUTE_B_MAX_K, K % 16 == 0. One wave on `stream`.
 * Returns GEMM_W4A4_EINVAL (NULL pointer, K out of range), GEMM_W4A4_EALIGN,
 * GEMM_W4A4_EDEVICE, GEMM_W4A4_ELAUNCH or GEMM_W4A4_OK.
 */
#define W4A4_PROBE_ROUTE_B_MAX_K 65536
int w4a4_probe_route_b_tile(const uint8_t* act, const uint8_t* ascales, const uint8_t* wgt,
                           const uint8_t* wscales, float* out, int K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_PROBES_H */
