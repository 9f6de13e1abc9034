"""ctypes view of libw4a4_probes.so (include/w4a4_probes.h): measurement aids
beside the operator, not part of it — the attainable rate of each matrix
instruction under full-chip load, and the two candidate routes of NVFP4's
block-scaled product on gfx950's matrix cores. Loads fail loudly if the
library has not been built."""
from __future__ import annotations

import ctypes
import os
import threading

from .build import PROBES_LIB_PATH

PEAK_GROUPS = 256                              # W4A4_PROBE_GROUPS
PEAK_FLOP = {0: 32768, 1: 131072, 2: 32768}    # per MFMA of each w4a4_probe_mfma_peak kind
ROUTE_FLOP_PER_BLOCK = 12 * 32768              # useful flop per wave and 16-k block, either route
ROUTE_B_MAX_K = 65536                          # W4A4_PROBE_ROUTE_B_MAX_K

_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return PROBES_LIB_PATH


def load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(PROBES_LIB_PATH):
            raise RuntimeError(f"{PROBES_LIB_PATH} is missing: build it first "
                               "(python -m bit_quantized_gemm_amd.build)")
        lib = ctypes.CDLL(PROBES_LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        lib.w4a4_probe_mfma_peak.argtypes = [i, i, vp, vp]
        lib.w4a4_probe_mfma_peak.restype = i
        lib.w4a4_probe_route_core.argtypes = [i, i, vp, vp]
        lib.w4a4_probe_route_core.restype = i
        lib.w4a4_probe_route_b_tile.argtypes = [vp] * 5 + [i, vp]
        lib.w4a4_probe_route_b_tile.restype = i
        _lib = lib
        return lib


def mfma_peak_raw(kind: int, iters: int, clocks, stream) -> int:
    """Launch the attainable-MFMA-rate microbenchmark; returns its code."""
    return load().w4a4_probe_mfma_peak(kind, iters, clocks, stream)


def route_core_raw(route: int, blocks: int, clocks, stream) -> int:
    """Launch the per-block arithmetic of route 0 (decode + fp16 MFMA) or
    route 1 (scaled FP4 MFMA + scale on partials) on every SIMD."""
    return load().w4a4_probe_route_core(route, blocks, clocks, stream)


def route_b_tile_raw(act, ascales, wgt, wscales, out, K: int, stream) -> int:
    """One 32x32 NVFP4 tile by route 1 into float32 `out`."""
    return load().w4a4_probe_route_b_tile(act, ascales, wgt, wscales, out, K, stream)
