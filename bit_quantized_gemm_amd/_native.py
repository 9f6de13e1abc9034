"""ctypes view of the C ABI declared in include/gemm_w4a4.h.

Only argument marshalling lives here: every step of the operator runs in the
HIP kernels of libgemm_w4a4.so. There is no fallback; if the library is
missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

OK = 0
EINVAL = -1
EALIGN = -2
ELAUNCH = -3
EOVERLAP = -4
EDEVICE = -5
ENOMEM = -6
ESCRATCH = -7
MAX_R = 1024

_PLAN_FIELDS = ("variant", "block_m", "block_n", "block_k", "stages", "waves_m", "waves_n",
                "threads", "lds_bytes", "lds_stage_bytes", "lds_limit", "tiles_m", "tiles_n",
                "grid", "k_stages", "lora_steps", "occupancy", "policy", "lora_place",
                "lds_ring_bytes", "lds_side_bytes", "flavour", "vgprs", "agprs", "sgprs",
                "regs_limit", "k_groups", "tail_variant", "tail_rows", "tail_block_m", "tail_block_n",
                "tail_grid", "tail_splits")


_QPLAN_FIELDS = ("variant", "wide", "rank_tiles", "rows", "threads", "lds_bytes", "row_blocks", "k_slices",
                 "spans_per_slice", "grid", "launches")


class QuantizePlan(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in _QPLAN_FIELDS] + [("scratch_bytes", ctypes.c_longlong)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f in _QPLAN_FIELDS + ("scratch_bytes",)}


class Plan(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in _PLAN_FIELDS]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f in _PLAN_FIELDS}


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load libgemm_w4a4.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m bit_quantized_gemm_amd.build "
                "or __graft_entry__.build()); there is no non-HIP fallback")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        lib.gemm_w4a4.argtypes = [vp] * 9 + [i, i, i, i, vp]
        lib.gemm_w4a4.restype = i
        lib.gemm_w4a4_f16.argtypes = [vp] * 9 + [i, i, i, i, vp]
        lib.gemm_w4a4_f16.restype = i
        lib.gemm_w4a4_plan.argtypes = [i, i, i, i, ctypes.POINTER(Plan)]
        lib.gemm_w4a4_plan.restype = i
        lib.gemm_w4a4_num_variants.argtypes = []
        lib.gemm_w4a4_num_variants.restype = i
        lib.gemm_w4a4_variant_info.argtypes = [i, ctypes.POINTER(Plan)]
        lib.gemm_w4a4_variant_info.restype = i
        for name in ("gemm_mxfp4", "gemm_mxfp4_f16"):
            getattr(lib, name).argtypes = [vp] * 9 + [i, i, i, i, vp]
            getattr(lib, name).restype = i
        lib.gemm_mxfp4_plan.argtypes = [i, i, i, i, ctypes.POINTER(Plan)]
        lib.gemm_mxfp4_plan.restype = i
        lib.gemm_mxfp4_num_variants.argtypes = []
        lib.gemm_mxfp4_num_variants.restype = i
        lib.gemm_mxfp4_variant_info.argtypes = [i, ctypes.POINTER(Plan)]
        lib.gemm_mxfp4_variant_info.restype = i
        lib.quantize_w4a4_act.argtypes = [vp] * 5 + [i, i, i, vp]
        lib.quantize_w4a4_act.restype = i
        lib.quantize_w4a4_act_noalloc.argtypes = [vp] * 5 + [i, i, i, vp]
        lib.quantize_w4a4_act_noalloc.restype = i
        lib.quantize_w4a4_act_plan.argtypes = [i, i, i, ctypes.POINTER(QuantizePlan)]
        lib.quantize_w4a4_act_plan.restype = i
        lib.gemm_w4a4_run.argtypes = [i, i, i] + [vp] * 9 + [i, i, i, i, vp]
        lib.gemm_w4a4_run.restype = i
        lib.gemm_w4a4_plan_variant.argtypes = [i, i, i, i, i, i, ctypes.POINTER(Plan)]
        lib.gemm_w4a4_plan_variant.restype = i
        lib.gemm_w4a4_strerror.argtypes = [i]
        lib.gemm_w4a4_strerror.restype = ctypes.c_char_p
        _lib = lib
        return lib


def strerror(code: int) -> str:
    return load().gemm_w4a4_strerror(code).decode()


def gemm_w4a4_raw(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                  M, N, K, R, stream) -> int:
    """Direct call of the C entry point with integer addresses; returns its code."""
    return load().gemm_w4a4(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                            out, M, N, K, R, stream)


def gemm_w4a4_f16_raw(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                      M, N, K, R, stream) -> int:
    """Direct call of the fp16 C entry point (LoRA and out in binary16); returns its code."""
    return load().gemm_w4a4_f16(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                                out, M, N, K, R, stream)


def gemm_mxfp4_raw(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                   M, N, K, R, stream) -> int:
    """Direct call of the MXFP4 C entry point (UE8M0 scales per 32 k); returns its code."""
    return load().gemm_mxfp4(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                             out, M, N, K, R, stream)


def gemm_mxfp4_f16_raw(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out,
                       M, N, K, R, stream) -> int:
    """Direct call of the MXFP4 fp16 C entry point; returns its code."""
    return load().gemm_mxfp4_f16(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                                 out, M, N, K, R, stream)


QUANTIZE_MAX_R = 128


def quantize_raw(x, lora_down, act, ascales, lora_act_in, M, K, R, stream) -> int:
    """Direct call of quantize_w4a4_act with integer addresses; returns its code."""
    return load().quantize_w4a4_act(x, lora_down, act, ascales, lora_act_in, M, K, R, stream)


def quantize_noalloc_raw(x, lora_down, act, ascales, lora_act_in, M, K, R, stream) -> int:
    """Direct call of quantize_w4a4_act_noalloc (no device allocation; its
    scratch is a fixed array per GPU) with integer addresses; returns its code."""
    return load().quantize_w4a4_act_noalloc(x, lora_down, act, ascales, lora_act_in, M, K, R, stream)


def quantize_plan(M: int, K: int, R: int) -> dict:
    """The launch quantize_w4a4_act would make for (M, K, R) (host only)."""
    p = QuantizePlan()
    rc = load().quantize_w4a4_act_plan(M, K, R, ctypes.byref(p))
    if rc != OK:
        raise ValueError(f"quantize_w4a4_act_plan: {strerror(rc)} ({rc})")
    return p.as_dict()


def run_raw(fmt: str, out_f16: bool, variant: int, act, ascales, wgt, wscales, wcscale, bias,
            lora_act_in, lora_up, out, M, N, K, R, stream) -> int:
    """gemm_w4a4_run: the operator with the format, output type and compiled
    instance (-1: the solver's choice) named explicitly; returns its code."""
    return load().gemm_w4a4_run(_FMT_CODE[fmt], int(out_f16), variant, act, ascales, wgt,
                                wscales, wcscale, bias, lora_act_in, lora_up, out, M, N, K, R,
                                stream)


def plan_variant(M: int, N: int, K: int, R: int, variant: int, fmt: str = "nvfp4") -> dict:
    """The plan of compiled instance `variant` (-1: the solver's) for a shape."""
    p = Plan()
    rc = load().gemm_w4a4_plan_variant(_FMT_CODE[fmt], variant, M, N, K, R, ctypes.byref(p))
    if rc != OK:
        raise ValueError(f"gemm_w4a4_plan_variant: {strerror(rc)} ({rc})")
    return p.as_dict()


_FMT_CODE = {"nvfp4": 0, "mxfp4": 1}
FORMATS = ("nvfp4", "mxfp4")
_PREFIX = {"nvfp4": "gemm_w4a4", "mxfp4": "gemm_mxfp4"}


def _fn(fmt: str, suffix: str):
    if fmt not in _PREFIX:
        raise ValueError(f"fmt must be one of {FORMATS}, got {fmt!r}")
    return getattr(load(), _PREFIX[fmt] + suffix)


def plan(M: int, N: int, K: int, R: int, fmt: str = "nvfp4") -> dict:
    p = Plan()
    rc = _fn(fmt, "_plan")(M, N, K, R, ctypes.byref(p))
    if rc != OK:
        raise ValueError(f"{_PREFIX[fmt]}_plan: {strerror(rc)} ({rc})")
    return p.as_dict()


def variants(fmt: str = "nvfp4") -> list:
    out = []
    info = _fn(fmt, "_variant_info")
    for v in range(_fn(fmt, "_num_variants")()):
        p = Plan()
        if info(v, ctypes.byref(p)) != OK:
            raise RuntimeError("variant_info failed")
        out.append(p.as_dict())
    return out
