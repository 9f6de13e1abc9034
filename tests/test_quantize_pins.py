"""Pins of the producer oracle (oracle/quantize_ref.py) to facts outside it (CPU only).

The oracle quantises bf16 activations to NVFP4 (E4M3 scale per 16 values,
E2M1 codes) and computes the LoRA-down product. Pinned against: hand-derived
golden blocks (tests/golden/nvfp4_quantize_cases.txt), an exact rational brute
force with its own grids (golden E2M1 table, torch's E4M3 decoder), torch's
own float32 -> E4M3FN cast for every bf16 amax, and properties that hold for
any correct quantiser: grid values round-trip, every code is a nearest grid
point, re-quantising a quantised block with a normal scale changes nothing.
A mutation test plants plausible mistakes and checks that a pin catches each.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.quantize_ref as qref
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                parts = line.split()
                vals[int(parts[0])] = float(parts[4])
    return vals


_E2M1 = _golden_e2m1()
_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16_bits(vals):
    """float64 values -> bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.tensor(np.asarray(vals, dtype=np.float64), dtype=torch.float64).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


def _nearest_even(v: Fraction, grid):
    """Index of the grid value nearest to v (grid increasing), ties to even, saturating."""
    best = None
    for i, g in enumerate(grid):
        d = abs(v - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


_E4M3_GRID = [float(_E4M3[b]) for b in range(0x7F)]
_E2M1_GRID = [_E2M1[c] for c in range(8)]


def brute_block(vals):
    """(scale byte, codes) of one block by exact rational search over the grids."""
    if any(not math.isfinite(v) for v in vals):
        return 0x7F, [0] * len(vals)
    amax = max(abs(Fraction(v)) for v in vals)
    sb = _nearest_even(amax / 6, _E4M3_GRID)
    s = Fraction(_E4M3_GRID[sb])
    codes = []
    for v in vals:
        mag = 0 if s == 0 else _nearest_even(abs(Fraction(v)) / s, _E2M1_GRID)
        codes.append((8 if math.copysign(1.0, v) < 0 else 0) | mag)
    return sb, codes


def brute_quantize(x_bits):
    x = _bits_to_f64(x_bits)
    M, K = x.shape
    act = np.zeros((M, K // 2), np.uint8)
    asc = np.zeros((K // 16, M), np.uint8)
    for m in range(M):
        for b in range(K // 16):
            sb, codes = brute_block(list(x[m, 16 * b:16 * b + 16]))
            asc[b, m] = sb
            for j in range(8):
                act[m, 8 * b + j] = codes[2 * j] | (codes[2 * j + 1] << 4)
    return act, asc


def _codes_of(act):
    c = np.empty((act.shape[0], 2 * act.shape[1]), np.uint8)
    c[:, 0::2] = act & 15
    c[:, 1::2] = act >> 4
    return c


# ------------------------------------------------------------ pins

def pin_golden_blocks():
    with open(os.path.join(GOLDEN, "nvfp4_quantize_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            vals_e, sb_e, codes_e = [p.strip() for p in line.split(";")[:3]]
            vals = [eval(v, {"__builtins__": {}, "float": float}) for v in vals_e.split(",")]
            vals += [0.0] * (16 - len(vals))
            bits = _bf16_bits(vals).reshape(1, 16)
            act, asc = qref.quantize_nvfp4_ref(bits)
            assert int(asc[0, 0]) == int(sb_e, 16), (vals_e, hex(asc[0, 0]), sb_e)
            got = "".join("%X" % c for c in _codes_of(act)[0])
            assert got == codes_e, (vals_e, got, codes_e)


def pin_bruteforce_random():
    """Vectorised oracle == exact rational search, on random blocks spanning
    many binades plus planted ties, zeros, signed zeros and non-finite values."""
    rng = np.random.default_rng(31)
    M, K = 12, 64
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-14, 12, size=(M, 1)))
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, 3] = np.nan
    x[3, 20] = np.inf
    x[4, :16] = np.array([6, 3, 1.5, 0.75, 0.25, 5, 2.5, 3.5, 1.25, 1.75, 0.5, 4, 1, 2, 0, 0])
    x[5, 16:32] = x[4, :16] * 1.125          # the same ties under a 1.125 scale
    x[6, :] = 1e30                            # scale saturates at 448
    x[7, :] = 1e-5                            # scale rounds to zero
    bits = _bf16_bits(x)
    want = brute_quantize(bits)
    got = qref.quantize_nvfp4_ref(bits)
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0], want[0])


def pin_scale_every_bf16_amax():
    """For every positive finite bf16 amax the scale byte equals torch's own
    float32 -> float8_e4m3fn cast of amax/6 (round to nearest even; the float32
    quotient sits on the same side of every E4M3 midpoint as the exact one),
    and the saturated value 448 where amax/6 exceeds it."""
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)          # all positive finite bf16
    amax = _bits_to_f64(bits)
    got = qref.e4m3_rne_bytes(amax)
    q = torch.from_numpy(amax).to(torch.float32) / 6.0
    inrange = (q <= 448.0).numpy()
    want = q.clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inrange], want[inrange])
    assert np.all(got[~inrange] == 0x7E)


def pin_round_trip_of_grid_values():
    """A block whose values are E2M1 values times a normal E4M3 scale s and
    whose largest magnitude is 6 s quantises to exactly that scale and those codes."""
    rng = np.random.default_rng(32)
    for sb in range(0x08, 0x7F, 3):
        s = _E4M3[sb]
        codes = rng.integers(0, 16, size=16)
        codes[rng.integers(16)] = 7 | (8 * rng.integers(2))
        vals = np.array([_E2M1[c] for c in codes]) * s
        if not np.all(np.abs(vals) < 3.3e38):
            continue
        bits = _bf16_bits(vals).reshape(1, 16)
        if not np.array_equal(_bits_to_f64(bits)[0], vals):
            continue                           # not exact in bf16 (very large scales)
        act, asc = qref.quantize_nvfp4_ref(bits)
        assert asc[0, 0] == sb, (sb, asc[0, 0])
        assert np.array_equal(_codes_of(act)[0], codes.astype(np.uint8)), (sb, codes)


def pin_codes_are_nearest():
    """Every decoded value is a nearest point of the scaled E2M1 grid to its
    input (unless the input is past 6 s, where it saturates)."""
    ld = synthetic.producer_inputs(64, 256, 0, seed=33)
    act, asc = qref.quantize_nvfp4_ref(ld["x"])
    x = _bits_to_f64(ld["x"])
    dq = qref.dequantize_blocks(act, asc)
    s = np.repeat(_E4M3[asc].T, 16, axis=1)
    grid = np.array(_E2M1_GRID)
    best = np.abs(np.abs(x)[..., None] - grid[None, None, :] * s[..., None]).min(axis=-1)
    err = np.abs(x - dq)
    sat = np.abs(x) > 6 * s
    assert np.all(err[~sat] == best[~sat])
    assert np.all(np.abs(dq[sat]) == 6 * s[sat])
    assert np.all(np.signbit(dq) == np.signbit(x))


def pin_requantisation_is_idempotent():
    """Quantising the dequantised operand again gives the same bytes wherever
    the block scale is a normal E4M3 number (there the largest code is always
    6: amax / s lies in [5.65, 6] or saturates)."""
    ld = synthetic.producer_inputs(48, 512, 0, seed=34)
    act, asc = qref.quantize_nvfp4_ref(ld["x"])
    dq = qref.dequantize_blocks(act, asc)
    act2, asc2 = qref.quantize_nvfp4_ref(_bf16_bits(dq))
    normal = np.repeat((asc >= 0x08) & (asc < 0x7F), 1, axis=0)
    assert np.array_equal(asc2[normal], asc[normal])
    rows_blocks = np.repeat(normal.T, 8, axis=1)
    assert np.array_equal(act2[rows_blocks], act[rows_blocks])


def pin_low_nibble_is_even_k():
    x = np.zeros((1, 16))
    x[0, 0] = 6.0                              # even k -> low nibble
    x[0, 3] = -3.0                             # odd k -> high nibble of byte 1
    act, asc = qref.quantize_nvfp4_ref(_bf16_bits(x))
    assert act[0, 0] == 0x07 and act[0, 1] == 0xD0 and asc[0, 0] == 0x38


def pin_scale_layout():
    """Scale of (row m, block b) sits at ascales[b, m]: all ones (amax/6 = 1/6
    -> 1.375 x 2^-3, byte 0x23) except row 2, block 1 (amax 12 -> 2.0, 0x40)."""
    x = np.ones((4, 48))
    x[2, 16:32] = 12.0
    act, asc = qref.quantize_nvfp4_ref(_bf16_bits(x))
    want = np.full((3, 4), 0x23, np.uint8)
    want[1, 2] = 0x40
    assert np.array_equal(asc, want), asc


def pin_lora_down_bruteforce():
    """The float64 LoRA-down product and its term magnitude equal exact
    rational sums over k (tiny shapes)."""
    d = synthetic.producer_inputs(3, 48, 5, seed=35)
    y = qref.lora_down_ref(d["x"], d["lora_down"])
    T = qref.lora_down_term_magnitude(d["x"], d["lora_down"])
    x = _bits_to_f64(d["x"])
    ld = _bits_to_f64(d["lora_down"])
    for m in range(3):
        for r in range(5):
            exact = sum(Fraction(x[m, k]) * Fraction(ld[r, k]) for k in range(48))
            mag = sum(abs(Fraction(x[m, k]) * Fraction(ld[r, k])) for k in range(48))
            assert abs(Fraction(y[m, r]) - exact) <= Fraction(2) ** -40 * mag
            assert abs(Fraction(T[m, r]) - mag) <= Fraction(2) ** -40 * mag
    assert qref.lora_down_ref(d["x"], d["lora_down"][:0]).shape == (3, 0)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------ mutation test

def _mut_scale_amax_over_4(mp):
    orig = qref.nearest_even_index
    mp.setattr(qref, "e4m3_rne_bytes",
               lambda amax: orig(amax, qref.E4M3_FINITE_NONNEG, 4.0).astype(np.uint8))


def _mut_scale_truncated(mp):
    mp.setattr(qref, "e4m3_rne_bytes", lambda amax: np.maximum(
        np.searchsorted(qref.E4M3_FINITE_NONNEG * 6.0, amax, side="right") - 1, 0).astype(np.uint8))


def _mut_ties_away_from_zero(mp):
    orig = qref.nearest_even_index

    def bad(v, grid, scale=1.0):
        if grid is qref.E2M1_MAGNITUDES:
            mids = (grid[:-1] + grid[1:]) / 2.0
            th = np.multiply.outer(np.asarray(scale, np.float64), mids)
            return (np.asarray(v)[..., None] >= th).sum(axis=-1)
        return orig(v, grid, scale)
    mp.setattr(qref, "nearest_even_index", bad)


def _mut_e2m1_ties_down(mp):
    orig = qref.nearest_even_index

    def bad(v, grid, scale=1.0):
        if grid is qref.E2M1_MAGNITUDES:
            mids = (grid[:-1] + grid[1:]) / 2.0
            th = np.multiply.outer(np.asarray(scale, np.float64), mids)
            return (np.asarray(v)[..., None] > th).sum(axis=-1)
        return orig(v, grid, scale)
    mp.setattr(qref, "nearest_even_index", bad)


def _mut_nibbles_swapped(mp):
    orig = qref.quantize_nvfp4_ref

    def bad(x):
        act, asc = orig(x)
        return ((act >> 4) | (act << 4)).astype(np.uint8), asc
    mp.setattr(qref, "quantize_nvfp4_ref", bad)


def _mut_scales_row_major(mp):
    orig = qref.quantize_nvfp4_ref

    def bad(x):
        act, asc = orig(x)
        return act, np.ascontiguousarray(asc.T).reshape(asc.shape)
    mp.setattr(qref, "quantize_nvfp4_ref", bad)


def _mut_sign_dropped(mp):
    orig = qref.quantize_nvfp4_ref

    def bad(x):
        act, asc = orig(x)
        return (act & 0x77).astype(np.uint8), asc
    mp.setattr(qref, "quantize_nvfp4_ref", bad)


def _mut_no_saturation(mp):
    # codes past 6 wrap into the sign bit instead of saturating
    orig = qref.nearest_even_index

    def bad(v, grid, scale=1.0):
        r = orig(v, grid, scale)
        if grid is qref.E2M1_MAGNITUDES:
            over = np.asarray(v) > 7 * np.asarray(scale, np.float64)
            r = np.where(over, 8, r)
        return r
    mp.setattr(qref, "nearest_even_index", bad)


def _mut_nan_block_unhandled(mp):
    orig = qref.quantize_nvfp4_ref

    def bad(x):
        xb = np.asarray(x, np.uint16).copy()
        nonfinite = (xb & 0x7F80) == 0x7F80
        xb[nonfinite] = 0x3F80                 # treats NaN / inf as 1.0
        return orig(xb)
    mp.setattr(qref, "quantize_nvfp4_ref", bad)


def _mut_lora_down_transposed(mp):
    def bad(x_bits, ld_bits):
        x = qref.bf16_bits_to_f64(x_bits)
        ld = qref.bf16_bits_to_f64(ld_bits)
        return x @ ld.reshape(-1)[: ld.size].reshape(ld.shape[1], ld.shape[0])
    mp.setattr(qref, "lora_down_ref", bad)


MUTANTS = [v for k, v in sorted(globals().items()) if k.startswith("_mut_")]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    with monkeypatch.context() as mp:
        mutant(mp)
        failed = []
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
        assert failed, f"no pin caught {mutant.__name__}"
