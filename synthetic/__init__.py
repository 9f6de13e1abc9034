"""Seeded synthetic inputs for the fused NVFP4 W4A4 operator.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It only draws random bytes and numbers in the layouts the operator
takes; it holds none of the operator's arithmetic (no E2M1/E4M3 decode, no
products, no sums). Every array it returns is a plain numpy array on the host;
callers copy it to the device themselves.

Layouts (all dense, row-major, no padding):
  act          uint8  [M, K/2]   two E2M1 codes per byte, low nibble = even k
  ascales      uint8  [K/16, M]  FP8-E4M3 (OCP E4M3FN) bytes, one per 16 k
  wgt          uint8  [N, K/2]
  wscales      uint8  [K/16, N]
  wcscale      float32 [N]
  bias         float32 [N]
  lora_act_in  uint16 [M, R]     bfloat16 bit patterns
  lora_up      uint16 [R, N]     bfloat16 bit patterns

The operator, its packing ([rows, K/2] bytes of two E2M1 codes, [K/16, rows]
E4M3 scales) and the rank-R LoRA residual follow the SVDQuant W4A4 on
Blackwell page ("Blackwell 上的 SVDQuant W4A4 算子实现"), section 2. The
value distributions and shapes below are the workloads this repository
measures: diffusion-transformer linear layers with hidden size 3072 and MLP
width 12288.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "custom_inputs", "no_lora_affine",
           "bf16_bits_from_f32", "f16_bits_from_f32", "e4m3_scale_byte", "large_inputs",
           "producer_inputs", "producer_workload_inputs", "PRODUCER_SEED_OFFSET"]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape plus the distribution knobs that differ."""
    name: str
    M: int
    N: int
    K: int
    R: int
    seed: int
    lora_act_std: float = 0.1
    lora_up_std: float = 0.1
    zero_scale_frac: float = 0.0   # fraction of E4M3 scale bytes forced to 0x00
    zero_bias_frac: float = 0.0    # fraction of bias entries forced to 0.0
    notes: str = field(default="", compare=False)

    @property
    def shape(self):
        return (self.M, self.N, self.K, self.R)

    def flops(self) -> int:
        """Algorithmic flops of one call: 2MNK for the main product + 2MRN for LoRA."""
        return 2 * self.M * self.N * self.K + 2 * self.M * self.R * self.N


WORKLOADS = {
    "tiny": Workload("tiny", 256, 256, 512, 32, seed=1000,
                     notes="small case, several tiles"),
    "qkv": Workload("qkv", 4096, 3072, 3072, 32, seed=1001,
                    notes="QKV-like linear, 4096 tokens, hidden 3072"),
    "mlp_up": Workload("mlp_up", 4096, 12288, 3072, 32, seed=1002,
                       notes="MLP-up linear 3072 -> 12288"),
    "mlp_down": Workload("mlp_down", 4096, 3072, 12288, 128, seed=1003, lora_act_std=0.05,
                         notes="MLP-down linear 12288 -> 3072 at LoRA rank 128"),
    "ragged": Workload("ragged", 1000, 3072, 3072, 16, seed=1004, zero_scale_frac=0.10,
                       zero_bias_frac=0.01,
                       notes="M not a tile multiple; 10% zero scale blocks, 1% zero bias"),
    # The four production shapes the SVDQuant W4A4 on Blackwell page measures
    # (section 9, "calibration": 9.1 the plain block-scaled GEMM ceiling, 9.2
    # the per-shape MFU table; M = 4352, (K, N, R) below), with the same value
    # distributions as the workloads above.
    "prod_k3840_n3072": Workload("prod_k3840_n3072", 4352, 3072, 3840, 128, seed=1005,
                                 notes="production shape M=4352 K=3840 N=3072, R=128"),
    "prod_k3840_n15360": Workload("prod_k3840_n15360", 4352, 15360, 3840, 128, seed=1006,
                                  notes="production shape M=4352 K=3840 N=15360, R=128"),
    "prod_k15360_n3840": Workload("prod_k15360_n3840", 4352, 3840, 15360, 128, seed=1007,
                                  notes="production shape M=4352 K=15360 N=3840, R=128"),
    "prod_k10240_n3072": Workload("prod_k10240_n3072", 4352, 3072, 10240, 32, seed=1008,
                                  notes="production shape M=4352 K=10240 N=3072, R=32"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (input recipe only).

    Used to turn normal samples into the bf16 LoRA inputs. NaN never occurs here.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def e4m3_scale_byte(exp: np.ndarray, mant: np.ndarray) -> np.ndarray:
    """Byte of a positive normal E4M3FN number 2**exp * (1 + mant/8).

    exp in [-6, 8], mant in [0, 7] (exp 8 with mant 7 is the NaN code and is
    rejected). This writes the bit fields only; it never evaluates the value.
    """
    exp = np.asarray(exp, dtype=np.int64)
    mant = np.asarray(mant, dtype=np.int64)
    if np.any(exp < -6) or np.any(exp > 8) or np.any(mant < 0) or np.any(mant > 7):
        raise ValueError("exponent/mantissa out of the E4M3 normal range")
    if np.any((exp == 8) & (mant == 7)):
        raise ValueError("0x7F/0xFF is the E4M3FN NaN code")
    return (((exp + 7) << 3) | mant).astype(np.uint8)


def _packed_codes(rng: np.random.Generator, rows: int, K: int) -> np.ndarray:
    lo = rng.integers(0, 16, size=(rows, K // 2), dtype=np.uint8)  # even k
    hi = rng.integers(0, 16, size=(rows, K // 2), dtype=np.uint8)  # odd k
    return (lo | (hi << 4)).astype(np.uint8)


def _scales(rng: np.random.Generator, kblocks: int, rows: int, zero_frac: float) -> np.ndarray:
    # random power of two in [2^-4, 2^2] times a mantissa 1 + m/8, m uniform in 0..7
    e = rng.integers(-4, 3, size=(kblocks, rows))
    m = rng.integers(0, 8, size=(kblocks, rows))
    s = e4m3_scale_byte(e, m)
    if zero_frac > 0.0:
        s[rng.random(size=s.shape) < zero_frac] = 0x00
    return s


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (numpy's nearest-even cast; input recipe only)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _e8m0_scales(rng: np.random.Generator, kblocks: int, rows: int, zero_frac: float) -> np.ndarray:
    # UE8M0 byte 127 + e: a power of two 2^e, e uniform in -4..2 (the NVFP4
    # recipe's exponent range; MX scales carry no mantissa). "Zero" blocks get
    # the smallest scale 2^-127 (byte 0x00): E8M0 has no zero.
    s = (127 + rng.integers(-4, 3, size=(kblocks, rows))).astype(np.uint8)
    if zero_frac > 0.0:
        s[rng.random(size=s.shape) < zero_frac] = 0x00
    return s


def make_inputs(wl: Workload | str, seed: int | None = None, dtype: str = "bf16",
                fmt: str = "nvfp4") -> dict:
    """Draw one seeded input set for a workload; returns a dict of numpy arrays.

    dtype ("bf16" or "f16") is the 16-bit type of the LoRA operands (and of
    the output the caller asks for); the draws are the same for both.
    fmt "nvfp4": E4M3 scales [K/16, rows]; "mxfp4": UE8M0 scales [K/32, rows]."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    M, N, K, R = wl.shape
    if K % 16 != 0:
        raise ValueError("K must be a multiple of 16")
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    if fmt not in ("nvfp4", "mxfp4"):
        raise ValueError("fmt must be nvfp4 or mxfp4")
    if fmt == "mxfp4" and K % 32:
        raise ValueError("MXFP4 needs K % 32 == 0")
    act = _packed_codes(rng, M, K)
    if fmt == "nvfp4":
        ascales = _scales(rng, K // 16, M, wl.zero_scale_frac)
    else:
        ascales = _e8m0_scales(rng, K // 32, M, wl.zero_scale_frac)
    wgt = _packed_codes(rng, N, K)
    if fmt == "nvfp4":
        wscales = _scales(rng, K // 16, N, wl.zero_scale_frac)
    else:
        wscales = _e8m0_scales(rng, K // 32, N, wl.zero_scale_frac)
    wcscale = rng.uniform(0.5, 1.5, size=N).astype(np.float32)
    bias = rng.standard_normal(size=N).astype(np.float32)
    if wl.zero_bias_frac > 0.0:
        bias[rng.random(size=N) < wl.zero_bias_frac] = 0.0
    if dtype not in ("bf16", "f16"):
        raise ValueError("dtype must be bf16 or f16")
    to_bits = bf16_bits_from_f32 if dtype == "bf16" else f16_bits_from_f32
    lora_act_in = to_bits((rng.standard_normal(size=(M, R)) * wl.lora_act_std).astype(np.float32))
    lora_up = to_bits((rng.standard_normal(size=(R, N)) * wl.lora_up_std).astype(np.float32))
    return dict(act=act, ascales=ascales, wgt=wgt, wscales=wscales, wcscale=wcscale,
                bias=bias, lora_act_in=lora_act_in, lora_up=lora_up, M=M, N=N, K=K, R=R,
                dtype=dtype, fmt=fmt)


def no_lora_affine(x: dict) -> dict:
    """The same packed operands and scales with the LoRA term and the affine
    switched off (R = 0, wcscale = 1, bias = 0): the plain block-scaled GEMM,
    the "ceiling" configuration the SVDQuant page compares against."""
    y = dict(x)
    M, N = x["M"], x["N"]
    y["R"] = 0
    y["lora_act_in"] = np.zeros((M, 0), np.uint16)
    y["lora_up"] = np.zeros((0, N), np.uint16)
    y["wcscale"] = np.ones(N, np.float32)
    y["bias"] = np.zeros(N, np.float32)
    return y


def custom_inputs(M: int, N: int, K: int, R: int, seed: int, dtype: str = "bf16",
                  fmt: str = "nvfp4", **kw) -> dict:
    """Inputs for an arbitrary shape with the standard distributions."""
    wl = Workload("custom", M, N, K, R, seed=seed, **kw)
    return make_inputs(wl, dtype=dtype, fmt=fmt)


def large_inputs(M: int, N: int, K: int, R: int, seed: int, fmt: str = "nvfp4") -> dict:
    """Inputs for shapes whose tensors approach 2^31 bytes, drawn byte-wise to
    keep host time and memory low: packed bytes uniform over 0..255 (so each
    nibble uniform over the 16 codes, independently), scale bytes as in
    make_inputs (E4M3 2^[-4,2] (1 + m/8), or UE8M0 2^[-4,2]), wcscale,
    bias and bf16 LoRA operands as in make_inputs."""
    rng = np.random.default_rng(seed)
    kb = K // (16 if fmt == "nvfp4" else 32)

    def scales(rows):
        if fmt == "nvfp4":
            e = rng.integers(3, 10, size=(kb, rows), dtype=np.uint8)   # biased exponent 7 + (-4..2)
            m = rng.integers(0, 8, size=(kb, rows), dtype=np.uint8)
            return (e << 3) | m
        return rng.integers(123, 130, size=(kb, rows), dtype=np.uint8)  # 127 + (-4..2)

    act = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    ascales = scales(M)
    wgt = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    wscales = scales(N)
    wcscale = rng.uniform(0.5, 1.5, size=N).astype(np.float32)
    bias = rng.standard_normal(size=N).astype(np.float32)
    lora_act_in = bf16_bits_from_f32((rng.standard_normal(size=(M, R)) * 0.1).astype(np.float32))
    lora_up = bf16_bits_from_f32((rng.standard_normal(size=(R, N)) * 0.1).astype(np.float32))
    return dict(act=act, ascales=ascales, wgt=wgt, wscales=wscales, wcscale=wcscale, bias=bias,
                lora_act_in=lora_act_in, lora_up=lora_up, M=M, N=N, K=K, R=R, dtype="bf16", fmt=fmt)


# ---------------------------------------------------------------- producer inputs
#
# The other half of the layer: bf16 activations x [M, K] (the tensor the fused
# GEMM's act / ascales are quantised from) and the LoRA-down weights
# lora_down [R, K] (one rank per row). The pages give no activation
# statistics; the recipe: x[m, k] = N(0, 1) * c[k] with a per-channel
# magnitude c[k] = 2^U(-3, 3) and 1 % of the channels 32x larger (outlier
# channels, the structure low-rank branches absorb), rounded to bf16;
# lora_down = bf16 of N(0, 0.02). The shapes are the GEMM workloads' M x K, R.

PRODUCER_SEED_OFFSET = 500


def producer_inputs(M: int, K: int, R: int, seed: int) -> dict:
    """Seeded producer inputs: x bf16 bits [M, K], lora_down bf16 bits [R, K]."""
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    rng = np.random.default_rng(seed)
    c = np.exp2(rng.uniform(-3.0, 3.0, size=K))
    c[rng.random(size=K) < 0.01] *= 32.0
    x = rng.standard_normal(size=(M, K)).astype(np.float32) * c.astype(np.float32)[None, :]
    lora_down = (rng.standard_normal(size=(R, K)) * 0.02).astype(np.float32)
    return dict(x=bf16_bits_from_f32(x), lora_down=bf16_bits_from_f32(lora_down), M=M, K=K, R=R)


def producer_workload_inputs(name: str) -> dict:
    """Producer inputs at a GEMM workload's M x K and rank R (the x it would quantise)."""
    wl = WORKLOADS[name]
    return producer_inputs(wl.M, wl.K, wl.R, seed=wl.seed + PRODUCER_SEED_OFFSET)
