"""Plain CPU oracle of the memory-bound half of SVDQuant W4A4: quantising the
activations to the fused GEMM's NVFP4 operand, and the LoRA-down product.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product
(``bit_quantized_gemm_amd``) never imports it and shares no code with it.

The SVDQuant W4A4 on Blackwell page ("Blackwell 上的 SVDQuant W4A4 算子实现",
section 1) calls the fused GEMM the compute-bound half of SVDQuant; this is the
half that produces its activation inputs. Section 2 fixes what it must emit:
act [M, K/2] (two E2M1 codes per byte, low nibble = even k in this
repository's reading), ascales [K/16, M] (one FP8-E4M3 scale per 16
consecutive k) and the rank-R LoRA input lora_act_in [M, R]; section 3.1 fixes
single-level scaling (no per-tensor factor). The pages give no rule for
choosing the scale or rounding the codes; the readings below are the plainest
that produce a valid NVFP4 operand (each is also listed in the design notes):

  * amax of a block = max |x| over its 16 values (x is bfloat16).
  * A block holding a NaN or an infinity gets the NaN scale byte 0x7F and
    all-zero codes (the GEMM then yields NaN for every output it touches).
  * scale byte = OCP E4M3FN round-to-nearest-even of amax / 6 (6 is the
    largest E2M1 magnitude), saturating at 448 (byte 0x7E).
  * With s the scale's value: code = sign bit of x (bit 3) | E2M1 magnitude of
    |x| / s rounded to nearest with ties to the even code, saturating at 6.
    When s is 0 (amax / 6 rounds to zero) every magnitude is 0 and only the
    sign bit is kept.
  * lora_act_in[m, r] = bf16 round-to-nearest-even of sum_k x[m, k] * lora_down[r, k],
    with lora_down stored [R, K] (one rank per row, k contiguous: the
    orientation of wgt).

Every rounding decision is taken on exact values: instead of dividing, amax is
compared with 6 x each midpoint of the E4M3 grid and |x| with s x each midpoint
of the E2M1 grid. Those products have at most 8 significant bits, so they are
exact in float64, as are all bf16 inputs; a comparison that comes out equal is
a tie and goes to the even neighbour.
"""
from __future__ import annotations

import numpy as np

from .w4a4_ref import E2M1_TABLE, E4M3_TABLE, bf16_bits_to_f64, bf16_rne_bits

__all__ = ["E2M1_MAGNITUDES", "E4M3_FINITE_NONNEG", "nearest_even_index", "e4m3_rne_bytes",
           "quantize_nvfp4_ref", "dequantize_blocks", "lora_down_ref", "lora_down_term_magnitude",
           "producer_ref"]

# E2M1 magnitudes by code 0..7 (bit 0 of a code is its mantissa bit, so even
# codes are the "even" neighbours of a tie).
E2M1_MAGNITUDES = np.array(E2M1_TABLE[:8], dtype=np.float64)
# Non-negative finite E4M3FN values by byte 0x00 .. 0x7E (0x7F is NaN); the
# byte's bit 0 is its mantissa bit.
E4M3_FINITE_NONNEG = np.array(E4M3_TABLE[:0x7F], dtype=np.float64)


def nearest_even_index(v: np.ndarray, grid: np.ndarray, scale=1.0) -> np.ndarray:
    """Index of the point of scale * grid nearest to each v >= 0; a tie goes to
    the even index; v past the last point saturates to it. `scale` is a
    power-of-two-free multiplier whose products with the grid's midpoints are
    exact in float64 (an E4M3 value, or 6)."""
    v = np.asarray(v, dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2.0                      # exact: at most 5 significant bits
    th = np.multiply.outer(np.asarray(scale, dtype=np.float64), mids)   # [..., len(grid)-1], exact
    vv = v[..., None]
    above = (vv > th).sum(axis=-1)
    tie_up = ((vv == th) & (np.arange(len(mids)) % 2 == 1)).sum(axis=-1)   # tie past an odd index
    return above + tie_up


def e4m3_rne_bytes(amax: np.ndarray) -> np.ndarray:
    """E4M3FN bytes of amax / 6 (amax >= 0, finite): nearest, ties to even, saturating at 0x7E."""
    return nearest_even_index(amax, E4M3_FINITE_NONNEG, 6.0).astype(np.uint8)


def quantize_nvfp4_ref(x_bits: np.ndarray):
    """x: bf16 bit patterns [M, K] (K % 16 == 0) -> (act uint8 [M, K/2],
    ascales uint8 [K/16, M]); the low nibble of each act byte is the even k."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    x = bf16_bits_to_f64(x_bits).reshape(M, K // 16, 16)   # [row, block, 16]
    finite = np.isfinite(x).all(axis=-1)                    # [row, block]
    ax = np.abs(np.where(np.isfinite(x), x, 0.0))
    amax = ax.max(axis=-1)
    sbyte = np.where(finite, e4m3_rne_bytes(amax), 0x7F).astype(np.uint8)
    s = np.where(finite, E4M3_FINITE_NONNEG[np.minimum(sbyte, 0x7E)], 0.0)   # [row, block]
    mag = nearest_even_index(ax, E2M1_MAGNITUDES, s[..., None])
    mag = np.where((s > 0)[..., None], mag, 0)
    sign = np.signbit(x).astype(np.int64) << 3
    codes = np.where(finite[..., None], sign | mag, 0).reshape(M, K).astype(np.uint8)
    act = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return act, np.ascontiguousarray(sbyte.T)


def dequantize_blocks(act: np.ndarray, ascales: np.ndarray) -> np.ndarray:
    """float64 values of an NVFP4 operand (act [M, K/2], ascales [K/16, M])."""
    M, half = act.shape
    codes = np.empty((M, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = act & 15
    codes[:, 1::2] = act >> 4
    return E2M1_TABLE[codes] * np.repeat(E4M3_TABLE[ascales].T, 16, axis=1)


def lora_down_ref(x_bits: np.ndarray, lora_down_bits: np.ndarray) -> np.ndarray:
    """float64 LoRA-down product [M, R]: sum_k x[m, k] * lora_down[r, k]."""
    x = bf16_bits_to_f64(x_bits)
    ld = bf16_bits_to_f64(lora_down_bits)
    if ld.shape[0] == 0:
        return np.zeros((x.shape[0], 0))
    return x @ ld.T


def lora_down_term_magnitude(x_bits: np.ndarray, lora_down_bits: np.ndarray) -> np.ndarray:
    """T[m, r] = sum_k |x[m, k] * lora_down[r, k]|: the scale of the acceptance bound."""
    x = np.abs(bf16_bits_to_f64(x_bits))
    ld = np.abs(bf16_bits_to_f64(lora_down_bits))
    if ld.shape[0] == 0:
        return np.zeros((x.shape[0], 0))
    return x @ ld.T


def producer_ref(x_bits, lora_down_bits):
    """(act, ascales, lora_act_in as float64, T) of the producer."""
    act, ascales = quantize_nvfp4_ref(x_bits)
    return act, ascales, lora_down_ref(x_bits, lora_down_bits), \
        lora_down_term_magnitude(x_bits, lora_down_bits)
