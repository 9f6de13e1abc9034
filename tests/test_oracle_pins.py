"""Pins of the CPU oracle to facts outside itself (CPU only).

Each pin ties the oracle to something it does not compute itself: golden values
derived by hand from the format definitions (tests/golden/), an independent
E4M3 decoder (torch.float8_e4m3fn), exact rational brute force on tiny inputs,
closed forms for structured inputs, and algebraic invariants. A mutation test
at the end plants plausible mistakes in the oracle and checks that at least one
pin fails for every one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.w4a4_ref as ref
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ARG_ORDER = ("act", "ascales", "wgt", "wscales", "wcscale", "bias", "lora_act_in", "lora_up")


def _args(x):
    return [x[k] for k in ARG_ORDER]


def _y(x):
    return ref.gemm_w4a4_ref(*_args(x))


# ------------------------------------------------------------ independent decoders

def _golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                parts = line.split()
                vals[int(parts[0])] = float(parts[4])
    return vals


def _torch_e4m3():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return b.to(torch.float64).numpy()


_E2M1_GOLD = _golden_e2m1()
_E4M3_TORCH = _torch_e4m3()


def _frac(x: float) -> Fraction:
    return Fraction(x)  # exact for every finite float


def brute_force(x) -> np.ndarray:
    """Exact y from element loops over rational numbers.

    Decodes with the golden E2M1 table and torch's E4M3 decoder, never with the
    oracle's tables, and walks every (m, n, k) and (m, n, r) one at a time.
    """
    M, N, K, R = x["M"], x["N"], x["K"], x["R"]
    act, wgt = x["act"], x["wgt"]
    asc, wsc = x["ascales"], x["wscales"]
    la = x["lora_act_in"].astype(np.uint32) << 16
    lu = x["lora_up"].astype(np.uint32) << 16
    la = la.view(np.float32)
    lu = lu.view(np.float32)
    y = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                byte_a = int(act[m, k // 2])
                byte_w = int(wgt[n, k // 2])
                ca = (byte_a >> 4) if (k % 2) else (byte_a & 15)
                cw = (byte_w >> 4) if (k % 2) else (byte_w & 15)
                a = _frac(_E2M1_GOLD[ca]) * _frac(_E4M3_TORCH[asc[k // 16, m]])
                w = _frac(_E2M1_GOLD[cw]) * _frac(_E4M3_TORCH[wsc[k // 16, n]])
                s += a * w
            lora = Fraction(0)
            for r in range(R):
                lora += _frac(float(la[m, r])) * _frac(float(lu[r, n]))
            y[m, n] = _frac(float(x["wcscale"][n])) * s + _frac(float(x["bias"][n])) + lora
    return y


def _small(M, N, K, R, seed, **kw):
    return synthetic.custom_inputs(M, N, K, R, seed=seed, **kw)


def _const_inputs(M, N, K, R, a_code, w_code, a_scale, w_scale, la_bits, lu_bits, seed=5):
    """Structured inputs: every nibble / scale / LoRA entry the same; wcscale, bias random."""
    rng = np.random.default_rng(seed)
    byte = lambda c: np.uint8(c | (c << 4))
    return dict(
        act=np.full((M, K // 2), byte(a_code), np.uint8),
        ascales=np.full((K // 16, M), a_scale, np.uint8),
        wgt=np.full((N, K // 2), byte(w_code), np.uint8),
        wscales=np.full((K // 16, N), w_scale, np.uint8),
        wcscale=rng.uniform(0.5, 1.5, N).astype(np.float32),
        bias=rng.standard_normal(N).astype(np.float32),
        lora_act_in=np.full((M, R), la_bits, np.uint16),
        lora_up=np.full((R, N), lu_bits, np.uint16),
        M=M, N=N, K=K, R=R)


# ------------------------------------------------------------ pins (return None or raise)

def pin_e2m1_golden():
    for c in range(16):
        v = ref.E2M1_TABLE[c]
        g = _E2M1_GOLD[c]
        assert v == g and math.copysign(1, v) == math.copysign(1, g), (c, v, g)


def pin_e4m3_torch():
    t = _E4M3_TORCH
    o = ref.E4M3_TABLE
    nan_t, nan_o = np.isnan(t), np.isnan(o)
    assert np.array_equal(nan_t, nan_o)
    assert np.array_equal(t[~nan_t], o[~nan_o])
    assert np.array_equal(np.signbit(t[~nan_t]), np.signbit(o[~nan_o]))


def pin_e4m3_golden():
    with open(os.path.join(GOLDEN, "e4m3_spot_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            b, v = line.split()
            b, v = int(b, 16), float(v)
            o = ref.E4M3_TABLE[b]
            if math.isnan(v):
                assert math.isnan(o), b
            else:
                assert o == v and math.copysign(1, o) == math.copysign(1, v), (hex(b), o, v)


def pin_bruteforce_tiny():
    """Vectorised oracle == exact rational loops on tiny random shapes (R in {0, 1, 3})."""
    for (M, N, K, R, seed) in [(3, 2, 16, 0, 1), (2, 3, 32, 1, 2), (4, 3, 48, 3, 3),
                               (1, 5, 32, 3, 4)]:
        x = _small(M, N, K, R, seed)
        y = _y(x)
        exact = brute_force(x)
        for m in range(M):
            for n in range(N):
                # float64 LoRA sums may round (random bf16 exponents); the main sum cannot
                assert abs(Fraction(y[m, n]) - exact[m, n]) <= Fraction(2) ** -40 * (
                    1 + abs(exact[m, n])), (M, N, K, R, m, n)


def pin_bruteforce_full_e4m3_range():
    """Scales drawn from every finite E4M3 byte (subnormals, 448, negative) still match."""
    rng = np.random.default_rng(11)
    x = _small(3, 4, 48, 2, 12)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    x["ascales"] = rng.choice(finite, size=x["ascales"].shape).astype(np.uint8)
    x["wscales"] = rng.choice(finite, size=x["wscales"].shape).astype(np.uint8)
    y = _y(x)
    exact = brute_force(x)
    for m in range(3):
        for n in range(4):
            assert abs(Fraction(y[m, n]) - exact[m, n]) <= Fraction(2) ** -44 * (
                1 + abs(exact[m, n])), (m, n)


def pin_exact_integer_accumulation():
    """Under the workload scales every product is a multiple of 2^-16, so the
    float64 main sum equals an int64 accumulation of (A*2^8)(W*2^8) exactly."""
    for name, rows in [("tiny", slice(0, 64)), ("qkv", slice(0, 16)), ("mlp_down", slice(0, 8))]:
        x = synthetic.make_inputs(name)
        act, asc = x["act"][rows], x["ascales"][:, rows]
        wgt, wsc = x["wgt"][:32], x["wscales"][:, :32]
        S = ref.main_product(act, asc, wgt, wsc)
        # integer decode straight from the bytes via the golden/torch tables
        def as_int(packed, scales):
            lo = packed & 15
            hi = packed >> 4
            codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)
            e2 = np.array([_E2M1_GOLD[c] for c in range(16)])[codes]
            sc = _E4M3_TORCH[scales].T.repeat(16, axis=1)
            v = e2 * sc * 256.0
            assert np.all(v == np.round(v))
            return v.astype(np.int64)
        ia = as_int(act, asc)
        iw = as_int(wgt, wsc)
        acc = ia @ iw.T                      # int64 matmul: exact
        assert np.array_equal(S * 65536.0, acc.astype(np.float64))
        assert np.all(np.abs(acc) < 2 ** 52)


def pin_closed_form_constant():
    """All nibbles and scales constant: y = K * a * sa * w * sw * wc[n] + bias[n] + R * la * lu."""
    cases = [
        # (a_code, w_code, a_scale, w_scale, a*sa*w*sw)
        (2, 2, 0x38, 0x38, 1.0),          # 1.0 * 1.0
        (5, 12, 0x40, 0x30, -6.0),        # (3 * 2) * (-2 * 0.5)
        (7, 9, 0x3F, 0x01, -6 * 1.875 * 0.5 * 2.0 ** -9),
    ]
    for (ac, wc_, asb, wsb, prod) in cases:
        M, N, K, R = 3, 5, 64, 4
        x = _const_inputs(M, N, K, R, ac, wc_, asb, wsb, 0x3F00, 0x3E80)   # 0.5, 0.25
        y = _y(x)
        wc = x["wcscale"].astype(np.float64)
        b = x["bias"].astype(np.float64)
        want = K * prod * wc + b + R * 0.5 * 0.25
        assert np.array_equal(y, np.broadcast_to(want, (M, N))), (ac, wc_)


def pin_nibble_order():
    """One nonzero act nibble: its byte's low half is k even, the high half k odd."""
    M, N, K, R = 4, 6, 64, 2
    rng = np.random.default_rng(21)
    for k0 in (18, 19, 0, 63):
        x = _const_inputs(M, N, K, R, 0, 0, 0x38, 0x38, 0x3F00, 0x3E80)
        m0, code = 2, 13                                   # -3.0
        x["act"][m0, k0 // 2] = code << (4 * (k0 % 2))
        # wgt: low nibbles 2.0, high nibbles 1.0, so the parity of k shows
        x["wgt"][:] = np.uint8(4 | (2 << 4))
        x["wscales"] = rng.choice([0x30, 0x38, 0x40, 0x48], size=x["wscales"].shape).astype(
            np.uint8)
        y = _y(x)
        sw = _E4M3_TORCH[x["wscales"][k0 // 16]]
        wparity = 2.0 if k0 % 2 == 0 else 1.0
        base = x["bias"].astype(np.float64) + R * 0.125
        want = np.tile(base, (M, 1))
        want[m0] += -3.0 * 1.0 * wparity * sw * x["wcscale"].astype(np.float64)
        assert np.array_equal(y, want), k0


def pin_scale_layout():
    """ascales is [K/16, M] and wscales [K/16, N]: a distinct scale moves one row / column only."""
    M, N, K, R = 5, 7, 96, 0
    for (kb0, m0, kb1, n1) in [(1, 3, 4, 2), (2, 0, 2, 6), (5, 4, 0, 0)]:
        x = _const_inputs(M, N, K, R, 2, 2, 0x38, 0x38, 0, 0)
        x["ascales"][kb0, m0] = 0x48     # 4.0
        x["wscales"][kb1, n1] = 0x30     # 0.5
        y = _y(x)
        sa = np.ones((K // 16, M))
        sa[kb0, m0] = 4.0
        sw = np.ones((K // 16, N))
        sw[kb1, n1] = 0.5
        S = 16.0 * (sa.T @ sw)           # sum over blocks of 16 * sa * sw
        want = S * x["wcscale"].astype(np.float64) + x["bias"].astype(np.float64)
        assert np.array_equal(y, want), (kb0, m0, kb1, n1)


def pin_r0_invariant():
    """R = 0 gives wc*S + bias; R > 0 with lora_up == 0 gives the very same values."""
    x = _small(6, 5, 64, 0, 31)
    y0 = _y(x)
    x1 = dict(x)
    x1["R"] = 3
    rng = np.random.default_rng(3)
    x1["lora_act_in"] = rng.integers(0, 0x7F00, size=(6, 3)).astype(np.uint16)
    x1["lora_up"] = np.zeros((3, 5), np.uint16)
    assert np.array_equal(_y(x1), y0)
    exact = brute_force(x)
    assert all(Fraction(y0[m, n]) == exact[m, n] for m in range(6) for n in range(5))


def pin_zero_main_term():
    """All act scales zero (or all act codes zero): y = bias + L, L from exact loops."""
    for mode in ("scales", "codes"):
        x = _small(4, 6, 32, 5, 41)
        if mode == "scales":
            x["ascales"][:] = 0
        else:
            x["act"][:] = 0
        y = _y(x)
        exact = brute_force(x)
        for m in range(4):
            for n in range(6):
                assert abs(Fraction(y[m, n]) - exact[m, n]) <= Fraction(2) ** -48, (mode, m, n)
        # and the LoRA term is visible: without it the result would differ
        assert not np.allclose(y, x["bias"].astype(np.float64)[None, :], atol=1e-6)


def pin_block_deletion():
    """Zeroing the scales of one k-block equals removing its 16 columns of k."""
    x = _small(5, 4, 80, 2, 51)
    for kb in (0, 2, 4):
        xz = dict(x)
        xz["ascales"] = x["ascales"].copy()
        xz["ascales"][kb] = 0
        keep_bytes = np.r_[0:kb * 8, (kb + 1) * 8:40]
        keep_blocks = np.r_[0:kb, kb + 1:5]
        xr = dict(x)
        xr["act"] = x["act"][:, keep_bytes].copy()
        xr["wgt"] = x["wgt"][:, keep_bytes].copy()
        xr["ascales"] = x["ascales"][keep_blocks].copy()
        xr["wscales"] = x["wscales"][keep_blocks].copy()
        xr["K"] = 64
        assert np.array_equal(_y(xz), _y(xr)), kb


def pin_linearity():
    """Doubling wcscale doubles the main term; raising every act scale exponent by one
    doubles S; adding c to bias adds c."""
    x = _small(6, 7, 64, 3, 61)
    y = _y(x)
    L = ref.lora_product(x["lora_act_in"], x["lora_up"])
    b = x["bias"].astype(np.float64)
    main = y - b - L
    x2 = dict(x)
    x2["wcscale"] = (x["wcscale"] * 2).astype(np.float32)
    assert np.allclose(_y(x2) - b - L, 2 * main, rtol=0, atol=1e-9 * np.abs(main).max())
    x3 = dict(x)
    x3["ascales"] = (x["ascales"] + 8).astype(np.uint8)      # exponent field + 1
    assert np.allclose(_y(x3) - b - L, 2 * main, rtol=0, atol=1e-9 * np.abs(main).max())
    x4 = dict(x)
    x4["bias"] = (x["bias"] + np.float32(0.75)).astype(np.float32)
    delta = x4["bias"].astype(np.float64) - b          # the fp32 sum rounds; use its real step
    assert np.allclose(_y(x4), y + delta[None, :], rtol=0, atol=1e-12 * np.abs(y).max())


def pin_transpose_symmetry():
    """With wc = 1, bias = 0, R = 0, swapping the two operands transposes y."""
    x = _small(5, 3, 48, 0, 71)
    x["wcscale"][:] = 1.0
    x["bias"][:] = 0.0
    y = _y(x)
    xt = dict(x)
    xt.update(act=x["wgt"], ascales=x["wscales"], wgt=x["act"], wscales=x["ascales"],
              wcscale=np.ones(5, np.float32), bias=np.zeros(5, np.float32),
              lora_act_in=np.zeros((3, 0), np.uint16), lora_up=np.zeros((0, 5), np.uint16),
              M=3, N=5)
    assert np.array_equal(_y(xt), y.T)


def pin_subnormal_scales():
    """Subnormal E4M3 scales (0x01..0x07): small main term, still exact."""
    x = _small(3, 4, 64, 2, 81)
    rng = np.random.default_rng(82)
    x["ascales"] = rng.integers(1, 8, size=x["ascales"].shape).astype(np.uint8)
    x["wscales"] = rng.integers(1, 8, size=x["wscales"].shape).astype(np.uint8)
    y = _y(x)
    exact = brute_force(x)
    for m in range(3):
        for n in range(4):
            assert abs(Fraction(y[m, n]) - exact[m, n]) <= Fraction(2) ** -48, (m, n)


def pin_bf16_rounding():
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            expr, bits, _ = [p.strip() for p in line.split(";")]
            v = eval(expr, {"__builtins__": {}})
            got = int(ref.bf16_rne_bits(np.array([v]))[0])
            assert got == int(bits, 16), (expr, hex(got), bits)
    # values exactly representable in float32 round the same way as torch's RNE cast
    rng = np.random.default_rng(91)
    f32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    tb = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref.bf16_rne_bits(f32.astype(np.float64)), tb)


def pin_ulp():
    u = ref.ulp_bf16(np.array([1.0, 1.5, 2.0, -3.0, 2.0 ** -126, 2.0 ** -130, 0.0, 255.0]))
    want = [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133,
            2.0 ** 0]
    assert list(u) == want


def pin_checker():
    """The acceptance check passes the rounded reference and catches a dropped LoRA or bias
    term on a case whose main term is zero."""
    x = _small(8, 8, 32, 4, 101)
    x["ascales"][:] = 0
    y = _y(x)
    T = ref.term_magnitude(*_args(x))
    assert ref.check_output(ref.bf16_rne_bits(y), y, T)["ok"]
    no_bias = y - x["bias"].astype(np.float64)[None, :]
    assert not ref.check_output(ref.bf16_rne_bits(no_bias), y, T)["ok"]
    no_lora = y - ref.lora_product(x["lora_act_in"], x["lora_up"])
    assert not ref.check_output(ref.bf16_rne_bits(no_lora), y, T)["ok"]


# ------------------------------------------------------------ the tolerance side: T, the bound, sampled rows

def brute_force_T(x, dtype="bf16"):
    """Exact T = |wc| * sum_k |a w| + |bias| + sum_r |la lu| from element loops over
    rational numbers (golden E2M1 table, torch's E4M3 / binary16 decoders), one
    (m, n, k) and (m, n, r) at a time; NVFP4 operands."""
    M, N, K, R = x["M"], x["N"], x["K"], x["R"]
    half = torch.float16 if dtype == "f16" else torch.bfloat16
    la = torch.from_numpy(x["lora_act_in"].view(np.int16)).view(half).to(torch.float64).numpy()
    lu = torch.from_numpy(x["lora_up"].view(np.int16)).view(half).to(torch.float64).numpy()
    T = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                ca = (int(x["act"][m, k // 2]) >> (4 * (k % 2))) & 15
                cw = (int(x["wgt"][n, k // 2]) >> (4 * (k % 2))) & 15
                a = _frac(_E2M1_GOLD[ca]) * _frac(_E4M3_TORCH[x["ascales"][k // 16, m]])
                w = _frac(_E2M1_GOLD[cw]) * _frac(_E4M3_TORCH[x["wscales"][k // 16, n]])
                s += abs(a * w)
            lora = Fraction(0)
            for r in range(R):
                lora += abs(_frac(float(la[m, r])) * _frac(float(lu[r, n])))
            T[m, n] = abs(_frac(float(x["wcscale"][n]))) * s + abs(_frac(float(x["bias"][n]))) + lora
    return T


def _assert_T_close(got, exact, what):
    # every term is >= 0, so the float64 sums only round (relative 2^-52 per addition)
    for idx in np.ndindex(*got.shape):
        assert abs(Fraction(float(got[idx])) - exact[idx]) <= Fraction(2) ** -40 * exact[idx], \
            (what, idx, float(got[idx]), float(exact[idx]))


def pin_term_magnitude_bruteforce():
    """term_magnitude == exact rational sum of |terms| on tiny shapes, with negative
    wcscale and bias, LoRA ranks 1 and 3, both 16-bit LoRA types."""
    for (M, N, K, R, seed, dtype) in [(3, 2, 32, 3, 21, "bf16"), (2, 4, 48, 1, 22, "bf16"),
                                      (4, 3, 32, 3, 23, "f16")]:
        x = synthetic.custom_inputs(M, N, K, R, seed=seed, dtype=dtype)
        x["wcscale"][0] = -x["wcscale"][0]          # |wcscale|, not wcscale
        x["bias"][:] = -np.abs(x["bias"])           # |bias|, not bias
        T = ref.term_magnitude(*_args(x), dtype=dtype)
        _assert_T_close(T, brute_force_T(x, dtype), (M, N, K, R, dtype))


def pin_term_magnitude_structured():
    """T for constant inputs in closed form: every main term is a*sa*w*sw (signs
    alternating over k, so the signed sum is 0 and T is not), plus |bias| and R|la lu|."""
    M, N, K, R = 3, 4, 32, 2
    x = _const_inputs(M, N, K, R, 2, 2, 0x38, 0x40, 0x3F00, 0xBE80)   # a=1, sa=1, w=1, sw=2
    x["act"][:] = 0xA2          # even k: +1.0, odd k: -1.0 (code 10 = -1.0)
    x["wcscale"][:] = -0.5
    T = ref.term_magnitude(*_args(x))
    y = _y(x)
    want_T = 0.5 * K * 2.0 + np.abs(x["bias"].astype(np.float64))[None, :] + R * 0.5 * 0.25
    assert np.array_equal(T, np.broadcast_to(want_T, (M, N))), (T, want_T)
    want_y = x["bias"].astype(np.float64)[None, :] + R * 0.5 * -0.25
    assert np.array_equal(y, np.broadcast_to(want_y, (M, N)))


def pin_tolerance_golden():
    """check_output's verdict on hand-derived cases at the edge of 4e-3*T + 1 ulp."""
    for row in _golden_rows("tolerance_cases.txt"):
        typ, y_e, T_e, got_e, verdict = row[:5]
        y_ref = float(eval(y_e, {"__builtins__": {}}))
        T = float(eval(T_e, {"__builtins__": {}}))
        got = float(eval(got_e, {"__builtins__": {}}))
        half = torch.float16 if typ == "f16" else torch.bfloat16
        g = torch.tensor([got], dtype=torch.float64).to(half)
        assert float(g.to(torch.float64)) == got, (got_e, "not exact in", typ)
        bits = g.view(torch.int16).numpy().view(np.uint16).reshape(1, 1)
        res = ref.check_output(bits, np.array([[y_ref]]), np.array([[T]]), typ)
        assert res["ok"] == (verdict == "pass"), (typ, y_e, T_e, got_e, verdict, res)


def pin_reference_rows():
    """The row-subset reference (used by full-size tests that sample rows) equals
    the full oracle's rows, both formats and both 16-bit types."""
    rows = np.array([0, 3, 4, 17, 30])
    for dtype in ("bf16", "f16"):
        x = synthetic.custom_inputs(31, 9, 64, 5, seed=24, dtype=dtype)
        x["dtype"] = dtype
        y, T = ref.reference_rows(x, rows)
        assert np.array_equal(y, ref.gemm_w4a4_ref(*_args(x), dtype=dtype)[rows])
        assert np.array_equal(T, ref.term_magnitude(*_args(x), dtype=dtype)[rows])
        xm = synthetic.custom_inputs(31, 9, 64, 5, seed=25, dtype=dtype, fmt="mxfp4")
        xm["dtype"] = dtype
        y, T = ref.reference_rows_mx(xm, rows)
        assert np.array_equal(y, ref.gemm_mxfp4_ref(*_args(xm), dtype=dtype)[rows])
        assert np.array_equal(T, ref.term_magnitude_mx(*_args(xm), dtype=dtype)[rows])


# ------------------------------------------------------------ fp16 variant (LoRA and output in binary16)

def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield [p.strip() for p in line.split(";")]


def pin_f16_decode():
    for bits, expr, _ in _golden_rows("f16_values.txt"):
        want = eval(expr, {"__builtins__": {}, "float": float})
        got = float(ref.f16_bits_to_f64(np.array([int(bits, 16)], np.uint16))[0])
        if math.isnan(want):
            assert math.isnan(got), bits
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (bits, got, want)
    # every one of the 65536 patterns against numpy's own binary16 type
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = ref.f16_bits_to_f64(allbits)
    npv = allbits.view(np.float16).astype(np.float64)
    nan = np.isnan(npv)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], npv[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(npv[~nan]))


def pin_f16_rounding():
    for expr, bits, _ in _golden_rows("f16_rounding.txt"):
        v = eval(expr, {"__builtins__": {}})
        got = int(ref.f16_rne_bits(np.array([v]))[0])
        assert got == int(bits, 16), (expr, hex(got), bits)
    # finite values from subnormal to overflow against numpy's float64 -> float16 cast
    rng = np.random.default_rng(92)
    v = rng.standard_normal(50000) * np.exp(rng.uniform(-20, 12, 50000))
    v = np.concatenate([v, rng.integers(-70000, 70000, 2000).astype(np.float64) + 0.5])
    with np.errstate(over="ignore"):
        npb = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ref.f16_rne_bits(v), npb)
    special = np.array([np.nan, np.inf, -np.inf])
    assert list(ref.f16_rne_bits(special)) == [0x7E00, 0x7C00, 0xFC00]


def pin_ulp_f16():
    u = ref.ulp_f16(np.array([1.0, 1.5, 2.0, -3.0, 2.0 ** -14, 2.0 ** -20, 0.0, 65504.0, 1000.0]))
    want = [2.0 ** -10, 2.0 ** -10, 2.0 ** -9, 2.0 ** -9, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24,
            32.0, 0.5]
    assert list(u) == want


def pin_f16_lora_closed_form():
    """fp16 LoRA operands: la = 0.5 (0x3800), lu = 0.25 (0x3400) -> the LoRA term is R/8."""
    M, N, K, R = 6, 10, 48, 5
    x = _const_inputs(M, N, K, R, 2, 2, 0x38, 0x38, 0x3800, 0x3400)
    y = ref.gemm_w4a4_ref(*_args(x), dtype="f16")
    want = K * 1.0 * x["wcscale"].astype(np.float64)[None, :] + x["bias"].astype(np.float64)[None, :] \
        + R * 0.125
    assert np.array_equal(y, np.broadcast_to(want, (M, N)))


def pin_checker_f16():
    """The fp16 check passes the rounded reference, catches a dropped LoRA or bias on a
    zero-main case, and accepts infinity only where the value overflows binary16."""
    x = synthetic.custom_inputs(8, 8, 32, 4, seed=103, dtype="f16")
    x["ascales"][:] = 0
    y = ref.gemm_w4a4_ref(*_args(x), dtype="f16")
    T = ref.term_magnitude(*_args(x), dtype="f16")
    assert ref.check_output(ref.f16_rne_bits(y), y, T, "f16")["ok"]
    no_bias = y - x["bias"].astype(np.float64)[None, :]
    assert not ref.check_output(ref.f16_rne_bits(no_bias), y, T, "f16")["ok"]
    no_lora = y - ref.lora_product(x["lora_act_in"], x["lora_up"], "f16")
    assert not ref.check_output(ref.f16_rne_bits(no_lora), y, T, "f16")["ok"]
    big = np.array([[70000.0, -70000.0, 60000.0]])
    Tb = np.abs(big)
    inf_bits = np.array([[0x7C00, 0xFC00, 0x7C00]], np.uint16)
    r = ref.check_output(inf_bits, big, Tb, "f16")
    assert r["n_fail"] == 1 and r["worst"] == (0, 2)   # 60000 + 240 < 65520: inf is wrong


# ------------------------------------------------------------ MXFP4 variant (UE8M0 per 32 k)

def _mx(M, N, K, R, seed, **kw):
    return synthetic.custom_inputs(M, N, K, R, seed=seed, fmt="mxfp4", **kw)


def _y_mx(x):
    return ref.gemm_mxfp4_ref(*_args(x))


def pin_e8m0_golden():
    for byte, expr, _ in _golden_rows("e8m0_values.txt"):
        want = eval(expr, {"__builtins__": {}, "float": float})
        got = ref.e8m0_value(int(byte, 16))
        assert (math.isnan(got) and math.isnan(want)) or got == want, (byte, got, want)


def pin_e8m0_torch():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    tv = t.to(torch.float64).numpy()
    nan = np.isnan(tv)
    assert np.array_equal(np.isnan(ref.E8M0_TABLE), nan)
    assert np.array_equal(ref.E8M0_TABLE[~nan], tv[~nan])


def brute_force_mx(x):
    """Exact rational evaluation with element loops and the golden E2M1 table;
    returns (y, T) as floats of the exact values."""
    e2m1 = _golden_e2m1()
    e8 = {b: Fraction(2) ** (b - 127) for b in range(255)}
    M, N, K, R = x["M"], x["N"], x["K"], x["R"]
    codes = lambda packed, r, k: (int(packed[r, k // 2]) >> (4 * (k % 2))) & 15
    la = ref.bf16_bits_to_f64(x["lora_act_in"])
    lu = ref.bf16_bits_to_f64(x["lora_up"])
    y = np.zeros((M, N))
    T = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = tot = Fraction(0)
            for k in range(K):
                a = _frac(e2m1[codes(x["act"], m, k)]) * e8[int(x["ascales"][k // 32, m])]
                w = _frac(e2m1[codes(x["wgt"], n, k)]) * e8[int(x["wscales"][k // 32, n])]
                acc += a * w
                tot += abs(a * w)
            lora = sum((_frac(la[m, r]) * _frac(lu[r, n]) for r in range(R)), Fraction(0))
            lora_abs = sum((abs(_frac(la[m, r]) * _frac(lu[r, n])) for r in range(R)), Fraction(0))
            wc = _frac(float(x["wcscale"][n]))
            y[m, n] = float(wc * acc + _frac(float(x["bias"][n])) + lora)
            T[m, n] = float(abs(wc) * tot + abs(_frac(float(x["bias"][n]))) + lora_abs)
    return y, T


def pin_mx_bruteforce_tiny():
    rng = np.random.default_rng(61)
    for (M, N, K, R) in [(3, 4, 32, 0), (5, 3, 64, 1), (4, 6, 96, 3)]:
        x = _mx(M, N, K, R, seed=int(rng.integers(1 << 30)))
        # exponents -7..7: every product is a multiple of 2^-16 below 2^20, so
        # the float64 sums are exact and must equal the rational values
        x["ascales"] = rng.integers(120, 135, size=x["ascales"].shape).astype(np.uint8)
        x["wscales"] = rng.integers(120, 135, size=x["wscales"].shape).astype(np.uint8)
        y, _ = brute_force_mx(x)
        assert np.array_equal(_y_mx(x), y), (M, N, K, R)
        # exponents over -31..32 and the smallest scale 2^-127: float64 sums
        # round; the oracle stays within K ulps of the exact value
        x["ascales"] = rng.integers(96, 160, size=x["ascales"].shape).astype(np.uint8)
        x["wscales"] = rng.integers(96, 160, size=x["wscales"].shape).astype(np.uint8)
        x["ascales"][0, 0] = 0
        y, T = brute_force_mx(x)
        assert np.all(np.abs(_y_mx(x) - y) <= 2.0 ** -45 * T), (M, N, K, R)


def pin_mx_term_magnitude_bruteforce():
    """term_magnitude_mx == the rational brute force's T (|wc| sum|a w| + |bias| +
    sum|la lu|), with negative wcscale and bias entries and R in {1, 3}."""
    rng = np.random.default_rng(66)
    for (M, N, K, R) in [(3, 4, 64, 3), (2, 3, 32, 1)]:
        x = _mx(M, N, K, R, seed=int(rng.integers(1 << 30)))
        x["ascales"] = rng.integers(120, 135, size=x["ascales"].shape).astype(np.uint8)
        x["wscales"] = rng.integers(120, 135, size=x["wscales"].shape).astype(np.uint8)
        x["wcscale"][0] = -x["wcscale"][0]
        x["bias"][:] = -np.abs(x["bias"])
        _, T = brute_force_mx(x)
        got = ref.term_magnitude_mx(*_args(x))
        assert np.all(np.abs(got - T) <= 2.0 ** -40 * T), (M, N, K, R, got, T)


def pin_mx_block_boundary():
    """k = 31 is scaled by block 0 and k = 32 by block 1, for act and for wgt."""
    M, N, K = 2, 3, 64
    for side, k in (("act", 31), ("act", 32), ("wgt", 31), ("wgt", 32)):
        x = _mx(M, N, K, 0, seed=62)
        x["act"][:] = 0x22 if side == "wgt" else 0
        x["wgt"][:] = 0x22 if side == "act" else 0
        x["ascales"][:] = 127
        x["wscales"][:] = 127
        x["wcscale"][:] = 1.0
        x["bias"][:] = 0.0
        pk = x[side]
        pk[0, k // 2] = (0x4 << (4 * (k % 2)))           # code 4 = 2.0 at (row 0, k)
        sc = "ascales" if side == "act" else "wscales"
        x[sc][1, 0] = 130                                 # block 1 of row 0 scaled by 8
        y = _y_mx(x)
        want = 2.0 * (8.0 if k >= 32 else 1.0)            # the other operand is all 1.0
        if side == "act":
            assert np.all(y[0] == want) and np.all(y[1] == 0), (side, k, y)
        else:
            assert np.all(y[:, 0] == want) and np.all(y[:, 1:] == 0), (side, k, y)


def pin_mx_closed_form():
    M, N, K, R = 3, 5, 96, 2
    x = _mx(M, N, K, R, seed=63)
    x["act"][:] = 0x77     # 6.0 everywhere
    x["wgt"][:] = 0x33     # 1.5 everywhere
    x["ascales"][:] = 125  # 2^-2
    x["wscales"][:] = 130  # 2^3
    x["lora_act_in"][:] = 0x3F00   # bf16 0.5
    x["lora_up"][:] = 0x3E80       # bf16 0.25
    y = _y_mx(x)
    want = K * 6.0 * 0.25 * 1.5 * 8.0 * x["wcscale"].astype(np.float64)[None, :] \
        + x["bias"].astype(np.float64)[None, :] + R * 0.125
    assert np.array_equal(y, np.broadcast_to(want, (M, N)))


def pin_mx_matches_nvfp4_where_both_apply():
    """An MXFP4 input whose scales are powers of two inside E4M3's range is also an
    NVFP4 input (each scale repeated for the two 16-k blocks of its 32): both
    oracles must agree exactly (the NVFP4 one is pinned independently above)."""
    x = _mx(17, 13, 192, 3, seed=64)
    nv = dict(x)
    e = x["ascales"].astype(np.int64) - 127
    nv["ascales"] = np.repeat(synthetic.e4m3_scale_byte(e, np.zeros_like(e)), 2, axis=0)
    e = x["wscales"].astype(np.int64) - 127
    nv["wscales"] = np.repeat(synthetic.e4m3_scale_byte(e, np.zeros_like(e)), 2, axis=0)
    assert np.array_equal(_y_mx(x), ref.gemm_w4a4_ref(*_args(nv)))
    assert np.array_equal(ref.term_magnitude_mx(*_args(x)), ref.term_magnitude(*_args(nv)))


def pin_mx_nan_scale():
    x = _mx(4, 4, 64, 0, seed=65)
    x["ascales"][1, 2] = 0xFF
    y = _y_mx(x)
    assert np.isnan(y[2]).all() and np.isfinite(np.delete(y, 2, 0)).all()


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------ mutation test

def _mut_nibble_swap_act_only(mp):
    # Swapping the nibble order in *both* operands permutes k the same way on
    # both sides and leaves y unchanged; the real mistake is a mismatch.
    orig = ref.unpack_codes
    def swapped(p):
        c = orig(p)
        return c.reshape(c.shape[0], -1, 2)[:, :, ::-1].reshape(c.shape)
    def bad(act, asc, wgt, wsc):
        codes = swapped(act)
        A = ref.E2M1_TABLE[codes] * np.repeat(ref.E4M3_TABLE[np.asarray(asc)].T, 16, axis=1)
        return A @ ref.dequantize(wgt, wsc).T
    mp.setattr(ref, "main_product", bad)


def _mut_scale_rows_as_blocks(mp):
    def bad(packed, scales):
        codes = ref.unpack_codes(packed)
        rows, K = codes.shape
        s = np.asarray(scales).reshape(-1)[: rows * (K // 16)].reshape(rows, K // 16)
        return ref.E2M1_TABLE[codes] * np.repeat(ref.E4M3_TABLE[s], 16, axis=1)
    mp.setattr(ref, "dequantize", bad)


def _mut_block32(mp):
    def bad(packed, scales):
        codes = ref.unpack_codes(packed)
        rows, K = codes.shape
        idx = np.minimum(np.arange(K) // 32, K // 16 - 1)
        return ref.E2M1_TABLE[codes] * ref.E4M3_TABLE[np.asarray(scales)[idx, :].T]
    mp.setattr(ref, "dequantize", bad)


def _mut_lora_scaled(mp):
    def bad(*a, dtype="bf16"):
        S = ref.main_product(*a[:4])
        wc = np.asarray(a[4], np.float64)
        return wc * (S + ref.lora_product(a[6], a[7], dtype)) + np.asarray(a[5], np.float64)
    mp.setattr(ref, "gemm_w4a4_ref", bad)


def _mut_drop_bias(mp):
    def bad(*a, dtype="bf16"):
        S = ref.main_product(*a[:4])
        return np.asarray(a[4], np.float64) * S + ref.lora_product(a[6], a[7], dtype)
    mp.setattr(ref, "gemm_w4a4_ref", bad)


def _mut_e2m1_unsigned(mp):
    mp.setattr(ref, "E2M1_TABLE", np.abs(ref.E2M1_TABLE))


def _mut_e2m1_subnormal(mp):
    t = ref.E2M1_TABLE.copy()
    t[1], t[9] = 0.75, -0.75
    mp.setattr(ref, "E2M1_TABLE", t)


def _mut_e4m3_bias8(mp):
    mp.setattr(ref, "E4M3_TABLE", ref.E4M3_TABLE / 2)


def _mut_e4m3_subnormal_as_normal(mp):
    t = ref.E4M3_TABLE.copy()
    for m in range(1, 8):
        t[m] = (1 + m / 8) * 2.0 ** -7
    mp.setattr(ref, "E4M3_TABLE", t)


def _mut_lora_up_transposed(mp):
    def bad(la, lu, dtype="bf16"):
        a = ref.half_bits_to_f64(la, dtype)
        u = ref.half_bits_to_f64(lu, dtype)
        if a.shape[1] == 0:
            return np.zeros((a.shape[0], u.shape[1]))
        # reads lora_up as if it were stored [N, R]
        ut = u.reshape(-1)[: u.size].reshape(u.shape[1], u.shape[0]).T
        return a @ ut
    mp.setattr(ref, "lora_product", bad)


def _mut_wgt_transposed_scales(mp):
    orig = ref.main_product
    def bad(act, asc, wgt, wsc):
        A = ref.dequantize(act, asc)
        wflip = np.asarray(wsc)[::-1].copy()    # blocks in reverse order
        W = ref.dequantize(wgt, wflip)
        return A @ W.T
    mp.setattr(ref, "main_product", bad)


def _mut_bf16_truncate(mp):
    def bad(y):
        y32 = np.asarray(y, np.float64).astype(np.float32)
        return (y32.view(np.uint32) >> 16).astype(np.uint16)
    mp.setattr(ref, "bf16_rne_bits", bad)


def _mut_f16_exponent_bias16(mp):
    orig = ref.f16_bits_to_f64
    mp.setattr(ref, "f16_bits_to_f64", lambda b: orig(b) / 2)


def _mut_f16_round_toward_zero(mp):
    orig = ref.f16_rne_bits
    def bad(y):
        y = np.asarray(y, np.float64)
        return orig(np.sign(y) * np.maximum(np.abs(y) - 0.49 * ref.ulp_f16(y), 0.0))
    mp.setattr(ref, "f16_rne_bits", bad)


def _mut_lora_type_ignored(mp):
    mp.setattr(ref, "half_bits_to_f64", lambda b, dtype="bf16": ref.bf16_bits_to_f64(b))


def _mut_mx_block16(mp):
    def bad(packed, scales):
        codes = ref.unpack_codes(packed)
        rows, K = codes.shape
        idx = np.minimum(np.arange(K) // 16, K // 32 - 1)
        return ref.E2M1_TABLE[codes] * ref.E8M0_TABLE[np.asarray(scales)[idx, :].T]
    mp.setattr(ref, "dequantize_mx", bad)


def _mut_e8m0_bias128(mp):
    mp.setattr(ref, "E8M0_TABLE", ref.E8M0_TABLE / 2)


def _mut_e8m0_nan_as_number(mp):
    t = ref.E8M0_TABLE.copy()
    t[255] = 2.0 ** 128
    mp.setattr(ref, "E8M0_TABLE", t)


def _mut_mx_scales_row_major(mp):
    def bad(packed, scales):
        codes = ref.unpack_codes(packed)
        rows, K = codes.shape
        s = np.asarray(scales).reshape(-1)[: rows * (K // 32)].reshape(rows, K // 32)
        return ref.E2M1_TABLE[codes] * np.repeat(ref.E8M0_TABLE[s], 32, axis=1)
    mp.setattr(ref, "dequantize_mx", bad)


# The tolerance side. A shared misreading would touch both formats at once, so
# each of these plants its mistake in the NVFP4 and the MXFP4 function together.

def _both_T(mp, wrap):
    for name in ("term_magnitude", "term_magnitude_mx"):
        orig = getattr(ref, name)
        mp.setattr(ref, name, wrap(orig))


def _mut_T_times8(mp):
    _both_T(mp, lambda f: (lambda *a, dtype="bf16": 8.0 * f(*a, dtype=dtype)))


def _mut_T_bias_twice(mp):
    _both_T(mp, lambda f: (lambda *a, dtype="bf16": f(*a, dtype=dtype)
                           + np.abs(np.asarray(a[5], np.float64))[None, :]))


def _mut_T_main_signed(mp):
    # |sum_k a w| instead of sum_k |a w|
    def wrap(f):
        def bad(act, asc, wgt, wsc, wc, b, la, lu, dtype="bf16"):
            deq = ref.dequantize if f is ref.term_magnitude else ref.dequantize_mx
            S = np.abs(deq(act, asc) @ deq(wgt, wsc).T)
            L = np.abs(ref.half_bits_to_f64(la, dtype)) @ np.abs(ref.half_bits_to_f64(lu, dtype)) \
                if np.asarray(la).shape[1] else 0.0
            return np.abs(np.asarray(wc, np.float64))[None, :] * S \
                + np.abs(np.asarray(b, np.float64))[None, :] + L
        return bad
    _both_T(mp, wrap)


def _mut_T_no_lora(mp):
    def wrap(f):
        def bad(act, asc, wgt, wsc, wc, b, la, lu, dtype="bf16"):
            z = np.zeros_like(np.asarray(la))[:, :0], np.zeros_like(np.asarray(lu))[:0, :]
            return f(act, asc, wgt, wsc, wc, b, *z, dtype=dtype)
        return bad
    _both_T(mp, wrap)


def _mut_tol_coefficient_4e2(mp):
    orig = ref.tolerance_bound
    mp.setattr(ref, "tolerance_bound", lambda y, T, dtype="bf16": orig(y, 10.0 * np.asarray(T), dtype))


def _mut_tol_no_ulp(mp):
    mp.setattr(ref, "tolerance_bound", lambda y, T, dtype="bf16": 4e-3 * np.asarray(T, np.float64))


def _mut_tol_two_ulps(mp):
    orig = ref.tolerance_bound
    ulp = {"bf16": ref.ulp_bf16, "f16": ref.ulp_f16}
    mp.setattr(ref, "tolerance_bound", lambda y, T, dtype="bf16": orig(y, T, dtype) + ulp[dtype](y))


def _mut_tol_bf16_ulp_always(mp):
    mp.setattr(ref, "tolerance_bound", lambda y, T, dtype="bf16": 4e-3 * np.asarray(T, np.float64)
               + ref.ulp_bf16(y))


def _mut_reference_rows_first_scales(mp):
    # takes the first len(rows) act-scale columns instead of the sampled rows' own
    def bad(inputs, rows):
        rows = np.asarray(rows, dtype=np.int64)
        args = (inputs["act"][rows], inputs["ascales"][:, :len(rows)], inputs["wgt"],
                inputs["wscales"], inputs["wcscale"], inputs["bias"], inputs["lora_act_in"][rows],
                inputs["lora_up"])
        dt = inputs.get("dtype", "bf16")
        return ref.gemm_w4a4_ref(*args, dtype=dt), ref.term_magnitude(*args, dtype=dt)
    mp.setattr(ref, "reference_rows", bad)


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
