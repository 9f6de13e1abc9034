"""Plain fp64 CPU oracle of the fused NVFP4 W4A4 operator.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product
(``bit_quantized_gemm_amd``) never imports it and shares no code with it.

What it computes, and where each step comes from:

  y[m, n] = wcscale[n] * sum_k A[m, k] * W[n, k]  +  bias[n]
            + sum_r lora_act_in[m, r] * lora_up[r, n]

  * The operator (one block-scaled FP4 product, one rank-R LoRA product and a
    per-column affine) and the input packing are stated in section 2 of the
    SVDQuant W4A4 on Blackwell page ("Blackwell 上的 SVDQuant W4A4 算子实现").
  * NVFP4 is E2M1 data with one FP8-E4M3 scale per 16 consecutive k and an
    fp32 accumulator; only this one level of scaling exists, any per-tensor
    factor having been folded into the block scales or wcscale (same page,
    section 3.1).
  * The per-column epilogue acc * wcscale[n] + bias[n] is the same page's
    section 6.6. LoRA is added after the wcscale product, as the operator
    formula in section 2 writes it.
  * E2M1 is one sign bit, two exponent bits and one mantissa bit (the DeepGEMM
    FP4 indexer page, "Step 0: 存储格式 → 逻辑值").

Readings where the pages are silent (each also listed in the design notes):
  low nibble of a byte holds the even k; wgt is [N, K/2]; the scale of (row, k)
  is scales[k // 16, row]; E4M3 is the OCP E4M3FN variant (bias 7, subnormals,
  NaN at S.1111.111, no infinities); wcscale and bias are fp32; R == 0 means no
  LoRA term.

The MXFP4 variant (second operator of this module, the *_mx functions):
  the same operator with OCP MX-scaled FP4 operands instead of NVFP4: E2M1
  codes as above, one UE8M0 scale per 32 consecutive k (an unsigned 8-bit
  power of two, 2^(b - 127), 0xFF = NaN, no zero). The DeepGEMM FP4 indexer
  page ("Step 0") describes this pairing, E2M1 data with a UE8M0 block scale
  that the matrix unit applies itself; its kernel shares one scale per 128
  elements, the MX block and gfx950's scaled MFMA use 32 (reading). Scales
  are laid out as for NVFP4: scales[k // 32, row].

Everything is evaluated in float64 after an exact decode. Every decoded value
has at most 6 significant bits and every product at most 12, so for the
synthetic workloads the main sum is exact in float64 whatever the summation
order (the pins in tests/ check this against exact rational arithmetic).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "e2m1_value", "e4m3_value", "E2M1_TABLE", "E4M3_TABLE", "unpack_codes", "dequantize",
    "bf16_bits_to_f64", "f16_bits_to_f64", "half_bits_to_f64", "main_product", "lora_product",
    "gemm_w4a4_ref", "term_magnitude", "bf16_rne_bits", "f16_rne_bits", "ulp_bf16", "ulp_f16",
    "tolerance_bound", "check_output", "validate", "HALF_TYPES",
    "e8m0_value", "E8M0_TABLE", "dequantize_mx", "gemm_mxfp4_ref", "term_magnitude_mx",
    "reference_rows_mx", "MX_BLOCK",
]

# The two 16-bit types the LoRA operands and the output may take. The
# SVDQuant page runs its operator with either ("c_dtype" fp16 or bf16, its
# sections 6.6 and 9.2); one call uses one type for lora_act_in, lora_up and out.
HALF_TYPES = ("bf16", "f16")


# ---------------------------------------------------------------- formats

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.

    Exponent field 0 is subnormal (0 or 0.5); there is no infinity or NaN.
    """
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code must be in 0..15")
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return sign * mag


def e4m3_value(byte: int) -> float:
    """Value of an OCP E4M3FN byte: sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities.
    """
    if not 0 <= byte <= 255:
        raise ValueError("E4M3 byte must be in 0..255")
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    exp = (byte >> 3) & 15
    man = byte & 7
    if exp == 15 and man == 7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] E2M1 codes; the low nibble is the even k."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of one NVFP4 operand.

    packed: [rows, K/2] uint8; scales: [K/16, rows] E4M3 bytes.
    Element (r, k) = E2M1(code[r, k]) * E4M3(scales[k // 16, r]).
    """
    codes = unpack_codes(packed)
    rows, K = codes.shape
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != (K // 16, rows):
        raise ValueError(f"scales shape {scales.shape} != {(K // 16, rows)}")
    vals = E2M1_TABLE[codes].reshape(rows, K // 16, 16)   # [row, k // 16, k % 16]
    per_block = E4M3_TABLE[scales].T                      # [row, k // 16]: scale of the block
    return (vals * per_block[:, :, None]).reshape(rows, K)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values.

    1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits; exponent field 0
    is zero/subnormal (m * 2^-24), field 31 is infinity (m = 0) or NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 31
    m = (b & 1023).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -24, np.ldexp(1.0 + m / 1024.0, e - 15))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def half_bits_to_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Bits of one of HALF_TYPES -> exact float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    raise ValueError(f"unknown 16-bit type {dtype!r}")


# ---------------------------------------------------------------- the operator

def validate(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up):
    """Shape and dtype checks; returns (M, N, K, R)."""
    act = np.asarray(act)
    wgt = np.asarray(wgt)
    if act.dtype != np.uint8 or wgt.dtype != np.uint8:
        raise ValueError("act and wgt must be uint8")
    if act.ndim != 2 or wgt.ndim != 2:
        raise ValueError("act and wgt must be 2-D")
    M, half = act.shape
    N = wgt.shape[0]
    K = 2 * half
    if wgt.shape[1] != half:
        raise ValueError("act and wgt must have the same K/2")
    if K % 16 != 0 or K == 0:
        raise ValueError("K must be a positive multiple of 16")
    if np.asarray(ascales).shape != (K // 16, M) or np.asarray(wscales).shape != (K // 16, N):
        raise ValueError("scale shapes must be [K/16, M] and [K/16, N]")
    if np.asarray(wcscale).shape != (N,) or np.asarray(bias).shape != (N,):
        raise ValueError("wcscale and bias must be [N]")
    la = np.asarray(lora_act_in)
    lu = np.asarray(lora_up)
    if la.ndim != 2 or lu.ndim != 2 or la.shape[0] != M or lu.shape[1] != N \
            or la.shape[1] != lu.shape[0]:
        raise ValueError("lora_act_in must be [M, R] and lora_up [R, N]")
    return M, N, K, la.shape[1]


def main_product(act, ascales, wgt, wscales) -> np.ndarray:
    """S[m, n] = sum_k A[m, k] * W[n, k] in float64 (a BLAS dgemm of exact values)."""
    A = dequantize(act, ascales)
    W = dequantize(wgt, wscales)
    return A @ W.T


def lora_product(lora_act_in, lora_up, dtype: str = "bf16") -> np.ndarray:
    """L[m, n] = sum_r lora_act_in[m, r] * lora_up[r, n] in float64."""
    la = half_bits_to_f64(lora_act_in, dtype)
    lu = half_bits_to_f64(lora_up, dtype)
    if la.shape[1] == 0:
        return np.zeros((la.shape[0], lu.shape[1]), dtype=np.float64)
    return la @ lu


def gemm_w4a4_ref(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                  dtype: str = "bf16") -> np.ndarray:
    """Reference result y (float64, [M, N]) of the fused operator; `dtype` is
    the 16-bit type (HALF_TYPES) of the LoRA operands."""
    validate(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up)
    S = main_product(act, ascales, wgt, wscales)
    wc = np.asarray(wcscale, dtype=np.float32).astype(np.float64)
    b = np.asarray(bias, dtype=np.float32).astype(np.float64)
    L = lora_product(lora_act_in, lora_up, dtype)
    return wc[None, :] * S + b[None, :] + L


def term_magnitude(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                   dtype: str = "bf16") -> np.ndarray:
    """T[m, n] = |wc[n]| sum_k |A W| + |bias[n]| + sum_r |la lu|: the scale of the tolerance."""
    A = np.abs(dequantize(act, ascales))
    W = np.abs(dequantize(wgt, wscales))
    wc = np.abs(np.asarray(wcscale, dtype=np.float32).astype(np.float64))
    b = np.abs(np.asarray(bias, dtype=np.float32).astype(np.float64))
    la = np.abs(half_bits_to_f64(lora_act_in, dtype))
    lu = np.abs(half_bits_to_f64(lora_up, dtype))
    L = la @ lu if la.shape[1] else np.zeros((la.shape[0], lu.shape[1]))
    return wc[None, :] * (A @ W.T) + b[None, :] + L


def reference_rows(inputs: dict, rows) -> tuple:
    """(y, T) for a subset of output rows only: the full-size parity tests sample rows."""
    rows = np.asarray(rows, dtype=np.int64)
    la = inputs["lora_act_in"][rows]
    args = (inputs["act"][rows], inputs["ascales"][:, rows], inputs["wgt"], inputs["wscales"],
            inputs["wcscale"], inputs["bias"], la, inputs["lora_up"])
    dtype = inputs.get("dtype", "bf16")
    return gemm_w4a4_ref(*args, dtype=dtype), term_magnitude(*args, dtype=dtype)


# ---------------------------------------------------------------- output rounding + tolerance

def bf16_rne_bits(y: np.ndarray) -> np.ndarray:
    """Round float64 values straight to bfloat16 (nearest, ties to even); returns uint16 bits.

    bf16 keeps 8 significant bits and fp32's exponent range: normal numbers
    from 2^-126, subnormals with spacing 2^-133. Rounding happens once, from
    float64 (no intermediate float32 rounding).
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, dtype=np.uint16)
    finite = np.isfinite(y)
    a = np.abs(np.where(finite, y, 0.0))
    _, e = np.frexp(a)                        # a = f * 2^e, f in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)           # spacing of bf16 numbers around a
    q = np.ldexp(1.0, q_exp)
    r = np.rint(a / q) * q                    # exact: division by a power of two; rint ties to even
    overflow = r >= 2.0 ** 128
    r32 = np.where(overflow, np.float32(np.inf), r).astype(np.float32)   # exact for r < 2^128
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.signbit(y) & finite, bits | np.uint16(0x8000), bits)
    out[finite] = bits[finite]
    out[np.isnan(y)] = 0x7FC0
    out[np.isposinf(y)] = 0x7F80
    out[np.isneginf(y)] = 0xFF80
    return out


def f16_rne_bits(y: np.ndarray) -> np.ndarray:
    """Round float64 values straight to IEEE binary16 (nearest, ties to even); uint16 bits.

    binary16 keeps 11 significant bits: normal numbers from 2^-14, subnormals
    with spacing 2^-24, largest finite 65504. A value at or above 65520 (the
    midpoint between 65504 and 2^16, a tie that goes to the even 2^16) becomes
    infinity. Rounding happens once, from float64.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, dtype=np.uint16)
    finite = np.isfinite(y)
    a = np.abs(np.where(finite, y, 0.0))
    _, e = np.frexp(a)                        # a = f * 2^e, f in [0.5, 1)
    q = np.ldexp(1.0, np.maximum(e - 11, -24))   # spacing of binary16 numbers around a
    r = np.rint(a / q) * q                    # exact: division by a power of two; rint ties to even
    overflow = r >= 2.0 ** 16
    # encode the (exactly representable) magnitude from its fields
    rs = np.where(overflow, 1.0, r)
    _, er = np.frexp(np.where(rs > 0, rs, 1.0))
    normal = rs >= 2.0 ** -14
    exp_field = np.where(normal, er - 1 + 15, 0)
    man = np.where(normal, rs / np.ldexp(1.0, er - 1) - 1.0, rs / 2.0 ** -24 / 1024.0) * 1024.0
    bits = (exp_field.astype(np.int64) << 10) | np.rint(man).astype(np.int64)
    bits = np.where(overflow, 0x7C00, np.where(rs > 0, bits, 0)).astype(np.uint16)
    bits = np.where(np.signbit(y) & finite, bits | np.uint16(0x8000), bits)
    out[finite] = bits[finite]
    out[np.isnan(y)] = 0x7E00
    out[np.isposinf(y)] = 0x7C00
    out[np.isneginf(y)] = 0xFC00
    return out


def ulp_f16(x: np.ndarray) -> np.ndarray:
    """Spacing of binary16 numbers at |x|: 2^(max(floor(log2|x|), -14) - 10); 2^-24 at 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))   # floor(log2 a) = e - 1
    u = np.ldexp(1.0, np.maximum(e - 1, -14) - 10)
    return np.where(a > 0, u, 2.0 ** -24)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x|: 2^(max(floor(log2|x|), -126) - 7); 2^-133 at 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))   # floor(log2 a) = e - 1
    u = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    return np.where(a > 0, u, 2.0 ** -133)


# Smallest magnitude that rounds to infinity under round-to-nearest-even.
OVERFLOW_AT = {"bf16": (2 - 2.0 ** -8) * 2.0 ** 127, "f16": 65520.0}


def tolerance_bound(y_ref: np.ndarray, T: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Per-element bound 4e-3 * T + one ulp of y_ref in the output type."""
    ulp = ulp_bf16 if dtype == "bf16" else ulp_f16
    return 4e-3 * np.asarray(T, dtype=np.float64) + ulp(y_ref)


def check_output(out_bits: np.ndarray, y_ref: np.ndarray, T: np.ndarray, dtype: str = "bf16") -> dict:
    """Compare output bits (type `dtype`) with the reference; NaN must match NaN.

    An infinite output is accepted only with the reference's sign and when the
    tolerance interval around the reference reaches the magnitude that rounds
    to infinity in that type (the output type cannot hold the value).
    Returns dict(ok, n_fail, max_ratio, worst) where ratio = |err| / bound.
    """
    got = half_bits_to_f64(out_bits, dtype)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    nan_ref = np.isnan(y_ref)
    nan_got = np.isnan(got)
    bound = tolerance_bound(np.where(nan_ref, 0.0, y_ref), np.where(nan_ref, 0.0, T), dtype)
    inf_got = np.isinf(got)
    inf_ok = inf_got & (np.sign(got) == np.sign(y_ref)) & \
        (np.abs(np.where(nan_ref, 0.0, y_ref)) + bound >= OVERFLOW_AT[dtype])
    err = np.abs(np.where(nan_ref | nan_got | inf_got, 0.0, got - y_ref))
    ratio = np.where(inf_got & ~inf_ok, np.inf, err / bound)
    fail = (ratio > 1.0) | (nan_ref != nan_got)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else None
    return dict(ok=not bool(fail.any()), n_fail=int(fail.sum()),
                max_ratio=float(ratio.max()) if ratio.size else 0.0, worst=worst)


# ---------------------------------------------------------------- MXFP4 variant

MX_BLOCK = 32   # k values per UE8M0 scale


def e8m0_value(b: int) -> float:
    """Value of a UE8M0 byte: 2^(b - 127); 0xFF is NaN (there is no zero or sign)."""
    if not 0 <= b <= 255:
        raise ValueError("E8M0 byte must be in 0..255")
    return math.nan if b == 255 else math.ldexp(1.0, b - 127)


E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def dequantize_mx(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of one MXFP4 operand.

    packed: [rows, K/2] uint8; scales: [K/32, rows] UE8M0 bytes.
    Element (r, k) = E2M1(code[r, k]) * E8M0(scales[k // 32, r]).
    """
    codes = unpack_codes(packed)
    rows, K = codes.shape
    scales = np.asarray(scales, dtype=np.uint8)
    if K % MX_BLOCK or scales.shape != (K // MX_BLOCK, rows):
        raise ValueError(f"scales shape {scales.shape} != {(K // MX_BLOCK, rows)}")
    vals = E2M1_TABLE[codes].reshape(rows, K // MX_BLOCK, MX_BLOCK)
    per_block = E8M0_TABLE[scales].T
    return (vals * per_block[:, :, None]).reshape(rows, K)


def gemm_mxfp4_ref(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                   dtype: str = "bf16") -> np.ndarray:
    """Reference y (float64, [M, N]) of the MXFP4 variant of the fused operator."""
    S = dequantize_mx(act, ascales) @ dequantize_mx(wgt, wscales).T
    wc = np.asarray(wcscale, dtype=np.float32).astype(np.float64)
    b = np.asarray(bias, dtype=np.float32).astype(np.float64)
    return wc[None, :] * S + b[None, :] + lora_product(lora_act_in, lora_up, dtype)


def term_magnitude_mx(act, ascales, wgt, wscales, wcscale, bias, lora_act_in, lora_up,
                      dtype: str = "bf16") -> np.ndarray:
    """T for the MXFP4 variant: |wc| sum_k |A W| + |bias| + sum_r |la lu|."""
    A = np.abs(dequantize_mx(act, ascales))
    W = np.abs(dequantize_mx(wgt, wscales))
    wc = np.abs(np.asarray(wcscale, dtype=np.float32).astype(np.float64))
    b = np.abs(np.asarray(bias, dtype=np.float32).astype(np.float64))
    la = np.abs(half_bits_to_f64(lora_act_in, dtype))
    lu = np.abs(half_bits_to_f64(lora_up, dtype))
    L = la @ lu if la.shape[1] else np.zeros((la.shape[0], lu.shape[1]))
    return wc[None, :] * (A @ W.T) + b[None, :] + L


def reference_rows_mx(inputs: dict, rows) -> tuple:
    """(y, T) of the MXFP4 variant for a subset of output rows."""
    rows = np.asarray(rows, dtype=np.int64)
    args = (inputs["act"][rows], inputs["ascales"][:, rows], inputs["wgt"], inputs["wscales"],
            inputs["wcscale"], inputs["bias"], inputs["lora_act_in"][rows], inputs["lora_up"])
    dtype = inputs.get("dtype", "bf16")
    return gemm_mxfp4_ref(*args, dtype=dtype), term_magnitude_mx(*args, dtype=dtype)
