"""Fused 4-bit W4A4 GEMM for AMD Instinct MI355X (gfx950).

    y = scaled_mma(act4, wgt4) * wcscale + bias + lora_act_in @ lora_up

with E2M1 operands and either NVFP4 block scales (FP8-E4M3, one per 16 k:
gemm_w4a4) or MXFP4 block scales (UE8M0, one per 32 k: gemm_mxfp4); and the
layer's other half, quantize_w4a4_act: bf16 activations -> the NVFP4 act /
ascales operand plus lora_act_in = x @ lora_down^T, in one pass over x.

Python binding over the C ABI of libgemm_w4a4.so (include/gemm_w4a4.h).
PyTorch supplies device memory and the stream; every step of the operator runs
in the library's HIP kernels. If the library is missing the calls raise.
"""
from __future__ import annotations

from . import _native
from ._native import (EALIGN, EDEVICE, EINVAL, ENOMEM, ESCRATCH, ELAUNCH, EOVERLAP, FORMATS, MAX_R, OK, QUANTIZE_MAX_R,
                      quantize_noalloc_raw, quantize_plan, quantize_raw,
                      gemm_mxfp4_f16_raw, gemm_mxfp4_raw, gemm_w4a4_f16_raw, gemm_w4a4_raw,
                      library_path, plan, plan_variant, run_raw, strerror, variants)

__all__ = ["gemm_w4a4", "gemm_mxfp4", "quantize_w4a4_act", "quantize_raw", "quantize_noalloc_raw", "quantize_plan", "QUANTIZE_MAX_R", "gemm_w4a4_raw", "gemm_w4a4_f16_raw", "gemm_mxfp4_raw",
           "gemm_mxfp4_f16_raw", "run_raw", "plan", "plan_variant", "variants", "strerror", "library_path", "GemmError", "OK",
           "EINVAL", "EALIGN", "ELAUNCH", "EOVERLAP", "EDEVICE", "ENOMEM", "ESCRATCH", "MAX_R", "FORMATS"]


class GemmError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"fused W4A4 GEMM failed: {strerror(code)} ({code})")
        self.code = code


def _check(t, name, dtype, shape, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gemm_w4a4(act, ascales, wgt, wscales, wcscale, bias, lora_act_in=None, lora_up=None,
              out=None, stream=None, dtype=None):
    """Enqueue the fused NVFP4 operator on `stream` (default: torch's current stream).

    act uint8 [M, K/2]; ascales uint8 (or float8_e4m3fn) [K/16, M];
    wgt uint8 [N, K/2]; wscales uint8 (or float8_e4m3fn) [K/16, N];
    wcscale, bias float32 [N]; lora_act_in [M, R] and lora_up [R, N] (both None
    for R = 0). Returns out [M, N] (allocated if None). The LoRA operands and
    out share one 16-bit type, torch.bfloat16 (gemm_w4a4) or torch.float16
    (gemm_w4a4_f16): `dtype`, else that of out, else of lora_act_in, else bf16.
    """
    return _launch("nvfp4", act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                   out, stream, dtype)


def gemm_mxfp4(act, ascales, wgt, wscales, wcscale, bias, lora_act_in=None, lora_up=None,
               out=None, stream=None, dtype=None):
    """Enqueue the fused MXFP4 operator on `stream`: as gemm_w4a4, but the
    block scales are UE8M0 bytes (2^(b-127); 255 = NaN), one per 32 k:
    ascales uint8 (or float8_e8m0fnu) [K/32, M], wscales [K/32, N]; K % 32 == 0.
    """
    return _launch("mxfp4", act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                   out, stream, dtype)


_BLOCK = {"nvfp4": 16, "mxfp4": 32}


def _launch(fmt, act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up, out, stream,
            dtype):
    import torch
    block = _BLOCK[fmt]
    if act.dim() != 2 or wgt.dim() != 2:
        raise ValueError("act and wgt must be 2-D")
    device = act.device
    if device.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    M, half = act.shape
    N = wgt.shape[0]
    K = 2 * half
    scale_dtype = torch.float8_e4m3fn if fmt == "nvfp4" else getattr(torch, "float8_e8m0fnu", None)
    if ascales.dtype == scale_dtype:
        ascales = ascales.view(torch.uint8)
    if wscales.dtype == scale_dtype:
        wscales = wscales.view(torch.uint8)
    _check(act, "act", torch.uint8, (M, half), device)
    _check(wgt, "wgt", torch.uint8, (N, half), device)
    _check(ascales, "ascales", torch.uint8, (K // block, M), device)
    _check(wscales, "wscales", torch.uint8, (K // block, N), device)
    _check(wcscale, "wcscale", torch.float32, (N,), device)
    _check(bias, "bias", torch.float32, (N,), device)
    if (lora_act_in is None) != (lora_up is None):
        raise ValueError("lora_act_in and lora_up go together")
    if dtype is None:
        dtype = out.dtype if out is not None else (
            lora_act_in.dtype if lora_act_in is not None else torch.bfloat16)
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"the LoRA/output type must be bfloat16 or float16, got {dtype}")
    if lora_act_in is None:
        R = 0
        la_ptr = lu_ptr = 0
    else:
        R = lora_act_in.shape[1]
        _check(lora_act_in, "lora_act_in", dtype, (M, R), device)
        _check(lora_up, "lora_up", dtype, (R, N), device)
        la_ptr, lu_ptr = lora_act_in.data_ptr(), lora_up.data_ptr()
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=device)
    _check(out, "out", dtype, (M, N), device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(device):
        f16 = dtype == torch.float16
        if fmt == "nvfp4":
            call = gemm_w4a4_f16_raw if f16 else gemm_w4a4_raw
        else:
            call = gemm_mxfp4_f16_raw if f16 else gemm_mxfp4_raw
        rc = call(act.data_ptr(), ascales.data_ptr(), wgt.data_ptr(), wscales.data_ptr(),
                  wcscale.data_ptr(), bias.data_ptr(), la_ptr, lu_ptr, out.data_ptr(), M, N, K, R,
                  handle)
    if rc != OK:
        raise GemmError(rc)
    return out


def quantize_w4a4_act(x, lora_down=None, act=None, ascales=None, lora_act_in=None, stream=None):
    """Enqueue the producer half on `stream`: x bfloat16 [M, K] (K % 16 == 0)
    -> act uint8 [M, K/2], ascales uint8 [K/16, M] (the NVFP4 operand of
    gemm_w4a4) and, when lora_down bfloat16 [R, K] is given, lora_act_in
    bfloat16 [M, R] = x @ lora_down^T. Outputs are allocated when None.
    Returns (act, ascales, lora_act_in or None)."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    device = x.device
    if device.type != "cuda":
        raise ValueError("tensors must live on a GPU device")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K), device)
    R = 0 if lora_down is None else lora_down.shape[0]
    if lora_down is not None:
        _check(lora_down, "lora_down", torch.bfloat16, (R, K), device)
    if act is None:
        act = torch.empty((M, K // 2), dtype=torch.uint8, device=device)
    if ascales is None:
        ascales = torch.empty((K // 16, M), dtype=torch.uint8, device=device)
    if R > 0 and lora_act_in is None:
        lora_act_in = torch.empty((M, R), dtype=torch.bfloat16, device=device)
    _check(act, "act", torch.uint8, (M, K // 2), device)
    _check(ascales, "ascales", torch.uint8, (K // 16, M), device)
    if R > 0:
        _check(lora_act_in, "lora_act_in", torch.bfloat16, (M, R), device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(device):
        rc = quantize_raw(x.data_ptr(), lora_down.data_ptr() if R else 0, act.data_ptr(),
                          ascales.data_ptr(), lora_act_in.data_ptr() if R else 0, M, K, R, handle)
    if rc != OK:
        raise GemmError(rc)
    return act, ascales, (lora_act_in if R else None)
