"""Parity of the HIP path (through the C ABI) with the CPU oracle. Needs a gfx950 GPU.

Acceptance per element: |y_gpu - y_ref| <= 4e-3 * T + 1 bf16 ulp(y_ref), with
T = |wcscale| sum_k |A W| + |bias| + sum_r |la lu| (oracle.check_output). Where
the exact result is representable in bf16 the check is bit-for-value exact.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_amd as w4
from bit_quantized_gemm_amd import probes
import oracle.w4a4_ref as ref
import synthetic

from gpu_helpers import ARGS, DEV, _say, assert_parity, full_reference, to_device

pytestmark = pytest.mark.gpu


def run_gpu(x, out=None):
    d = to_device(x)
    half = torch.float16 if x.get("dtype", "bf16") == "f16" else torch.bfloat16
    o = w4.gemm_w4a4(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
                     d["lora_act_in"], d["lora_up"], out=out, dtype=half)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_full(x):
    a = [x[k] for k in ARGS]
    dt = x.get("dtype", "bf16")
    return ref.gemm_w4a4_ref(*a, dtype=dt), ref.term_magnitude(*a, dtype=dt)


def const_inputs(M, N, K, R, a_code, w_code, a_scale, w_scale, la_bits=0x3F00, lu_bits=0x3E80,
                 seed=5):
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
        lora_up=np.full((R, N), lu_bits, np.uint16), M=M, N=N, K=K, R=R)


# ---------------------------------------------------------------- workloads

def test_tiny_full():
    _say("case: tiny workload 256x256x512 R=32, full comparison")
    x = synthetic.make_inputs("tiny")
    got = run_gpu(x)
    y, T = oracle_full(x)
    assert_parity(got, y, T, "tiny")


@pytest.mark.parametrize("name", ["qkv", "mlp_up", "mlp_down", "ragged", "prod_k3840_n3072",
                                  "prod_k3840_n15360", "prod_k15360_n3840", "prod_k10240_n3072"])
def test_workload_full_size(name):
    wl = synthetic.workload(name)
    _say(f"case: {name} {wl.shape}, full-size launch, every element vs oracle")
    x = synthetic.make_inputs(name)
    got = run_gpu(x)
    y, T = full_reference(x)
    assert_parity(got, y, T, f"{name} (all {wl.M} x {wl.N})")
    # every output is finite (no NaN scale bytes in these inputs)
    vals = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(vals).all()


@pytest.mark.parametrize("name", ["qkv", "prod_k3840_n3072"])
def test_ceiling_mode_full_size(name):
    """LoRA and affine off (R = 0, wcscale = 1, bias = 0) at full size."""
    wl = synthetic.workload(name)
    _say(f"case: {name} ceiling mode (no LoRA, no affine), every element vs oracle")
    x = synthetic.no_lora_affine(synthetic.make_inputs(name))
    got = run_gpu(x)
    y, T = full_reference(x)
    assert_parity(got, y, T, f"{name} ceiling (all {wl.M} x {wl.N})")


def test_deterministic_bytes():
    _say("case: determinism, ragged workload twice")
    x = synthetic.make_inputs("ragged")
    assert np.array_equal(run_gpu(x), run_gpu(x))


# ---------------------------------------------------------------- exhaustive decode

def _decode_case(side):
    """Every (E2M1 code, E4M3 byte) pair on one operand side, exact output expected."""
    rows = 16 * 256
    code = np.arange(rows) % 16
    sbyte = (np.arange(rows) // 16).astype(np.uint8)
    packed = (code | (code << 4)).astype(np.uint8)[:, None].repeat(8, axis=1)
    other = 64
    x = dict(K=16, R=0, lora_act_in=None, lora_up=None)
    one_packed = np.full((other, 8), 0x22, np.uint8)           # all 1.0
    one_scale = np.full((1, other), 0x38, np.uint8)            # 1.0
    if side == "act":
        x.update(M=rows, N=other, act=packed, ascales=sbyte[None, :], wgt=one_packed,
                 wscales=one_scale)
    else:
        x.update(M=other, N=rows, act=one_packed, ascales=one_scale, wgt=packed,
                 wscales=sbyte[None, :])
    x["wcscale"] = np.full(x["N"], 1 / 16, np.float32)          # 16 equal terms -> exact
    x["bias"] = np.zeros(x["N"], np.float32)
    x["lora_act_in"] = np.zeros((x["M"], 0), np.uint16)
    x["lora_up"] = np.zeros((0, x["N"]), np.uint16)
    return x


@pytest.mark.parametrize("side", ["act", "wgt"])
def test_decode_exhaustive(side):
    _say(f"case: exhaustive decode, {side} side, 16 codes x 256 scale bytes")
    x = _decode_case(side)
    got = run_gpu(x)
    y, T = oracle_full(x)
    gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan_y = np.isnan(y)
    assert np.array_equal(np.isnan(gv), nan_y)
    assert np.array_equal(gv[~nan_y], y[~nan_y])                # exact, value for value


# ---------------------------------------------------------------- structured probes

def test_probe_closed_form():
    _say("case: closed form, constant codes and scales, R=4")
    for (ac, wc_, asb, wsb) in [(2, 2, 0x38, 0x38), (5, 12, 0x40, 0x30), (7, 9, 0x3F, 0x01)]:
        x = const_inputs(300, 200, 256, 4, ac, wc_, asb, wsb)
        y, T = oracle_full(x)
        assert_parity(run_gpu(x), y, T, f"closed form {ac},{wc_}")


def test_probe_nibble_and_scale_layout():
    _say("case: single-nibble and single-scale probes")
    rng = np.random.default_rng(3)
    for k0 in (0, 19, 200, 255):
        x = const_inputs(70, 90, 256, 2, 0, 0, 0x38, 0x38)
        x["act"][33, k0 // 2] = 13 << (4 * (k0 % 2))
        x["wgt"][:] = np.uint8(4 | (2 << 4))
        x["wscales"] = rng.choice([0x30, 0x38, 0x40, 0x48], size=x["wscales"].shape).astype(
            np.uint8)
        y, T = oracle_full(x)
        assert_parity(run_gpu(x), y, T, f"nibble k0={k0}")
    for (kb0, m0, kb1, n1) in [(1, 3, 4, 2), (2, 250, 2, 190), (15, 299, 0, 0)]:
        x = const_inputs(300, 200, 256, 0, 2, 2, 0x38, 0x38)
        x["lora_act_in"] = np.zeros((300, 0), np.uint16)
        x["lora_up"] = np.zeros((0, 200), np.uint16)
        x["ascales"][kb0, m0] = 0x48
        x["wscales"][kb1, n1] = 0x30
        y, T = oracle_full(x)
        got = run_gpu(x)
        assert_parity(got, y, T, f"scale probe {(kb0, m0, kb1, n1)}")
        gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        # main term 16 * (integers) * wc: compare the rounded values exactly
        assert np.array_equal(gv, ref.bf16_bits_to_f64(ref.bf16_rne_bits(y)))


def test_probe_zero_main_term_shows_lora_and_bias():
    """All act scales zero: y = bias + LoRA, O(1), so a dropped or mis-scaled
    LoRA or bias term fails the tolerance."""
    _say("case: zero main term, LoRA + bias visible")
    for R in (1, 16, 32, 128, 3):
        x = synthetic.custom_inputs(260, 200, 256, R, seed=100 + R)
        x["ascales"][:] = 0
        y, T = oracle_full(x)
        got = run_gpu(x)
        assert_parity(got, y, T, f"zero main R={R}")
        # tighter than the tolerance: fp32 sum of at most R+1 terms
        gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.abs(gv - y) <= 2 * ref.ulp_bf16(y) + 1e-6)


# ranks past the pages' production bound (R <= 128) up to the library's
# limit: many 32-rank chunks, fast flavour (M, N, R multiples of 8, both
# 256-row and 128x128 tiles) and general (R % 8 != 0, M % 8 != 0)
LARGE_R = [(256, 200, 256, 160), (256, 192, 128, 1024), (64, 64, 64, 520), (260, 200, 256, 1000),
           # 256x192 tiles (their first chunk comes from the side region) and 256x128
           (4096, 3072, 128, 160), (4096, 3072, 128, 1024), (4352, 3072, 128, 256)]


@pytest.mark.parametrize("shape", LARGE_R, ids=["x".join(map(str, s)) for s in LARGE_R])
def test_probe_large_rank_lora_visible(shape):
    """Zero main term at large R: y = bias + a sum of R LoRA products, so a
    chunk dropped, repeated or read at the wrong ranks fails the check."""
    M, N, K, R = shape
    _say(f"case: zero main term at R={R}, M={M} N={N} K={K}")
    x = synthetic.custom_inputs(M, N, K, R, seed=500 + R)
    x["ascales"][:] = 0
    y, T = oracle_full(x)
    got = run_gpu(x)
    assert_parity(got, y, T, f"zero main R={R}")
    gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(gv - y) <= 2 * ref.ulp_bf16(y) + 1e-5)


def test_probe_subnormal_scales():
    _say("case: subnormal E4M3 scales, small main term")
    x = synthetic.custom_inputs(256, 192, 3072, 32, seed=9)
    rng = np.random.default_rng(10)
    x["ascales"] = rng.integers(1, 8, size=x["ascales"].shape).astype(np.uint8)
    x["wscales"] = rng.integers(1, 8, size=x["wscales"].shape).astype(np.uint8)
    y, T = oracle_full(x)
    assert_parity(run_gpu(x), y, T, "subnormal scales")


def test_probe_r0_equals_zero_lora_up():
    _say("case: R=0 (no LoRA pointers) equals R=16 with lora_up = 0")
    x = synthetic.custom_inputs(300, 260, 384, 16, seed=21)
    x0 = dict(x)
    x0["R"] = 0
    x0["lora_act_in"] = np.zeros((300, 0), np.uint16)
    x0["lora_up"] = np.zeros((0, 260), np.uint16)
    xz = dict(x)
    xz["lora_up"] = np.zeros_like(x["lora_up"])
    g0 = run_gpu(x0)
    assert np.array_equal(g0, run_gpu(xz))
    y, T = oracle_full(x0)
    assert_parity(g0, y, T, "R=0")


def test_probe_nan_scale_propagates():
    _say("case: NaN scale byte")
    x = synthetic.custom_inputs(64, 64, 64, 0, seed=31)
    x["ascales"][1, 5] = 0x7F
    x["wscales"][3, 9] = 0xFF
    got = run_gpu(x)
    y, T = oracle_full(x)
    assert_parity(got, y, T, "nan scale")
    gv = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.isnan(gv[5]).all() and np.isnan(gv[:, 9]).all()
    assert np.isfinite(np.delete(np.delete(gv, 5, 0), 9, 1)).all()


# ---------------------------------------------------------------- edge shapes

EDGE = [(1, 1, 16, 0), (1, 5, 16, 1), (7, 33, 48, 3), (33, 200, 144, 16), (257, 193, 272, 32),
        (300, 129, 160, 17), (64, 64, 4096, 128), (513, 385, 256, 128), (129, 1, 32, 8),
        (2, 1000, 112, 24), (1000, 64, 208, 40),
        # fast flavour (K % 32 == 0, M % 8 == 0, N % 8 == 0, R % 8 == 0):
        # edge tiles, several LoRA rank chunks, a last chunk only partly inside R
        (304, 200, 256, 40), (104, 3000, 512, 72), (136, 8, 32, 8), (64, 64, 384, 24),
        (256, 200, 640, 16), (512, 384, 1024, 0),
        # fast flavour with M % 8 != 0 (act scales in 12-byte windows), the
        # window clamped at the end of a tiny act-scale tensor; and M % 8 != 0
        # where the act-scale tensor size is not a multiple of 4 (general)
        (257, 200, 256, 32), (1001, 64, 128, 16), (259, 384, 512, 0), (3, 8, 64, 8), (5, 16, 64, 0),
        (7, 8, 32, 8), (1001, 64, 96, 16), (1, 8, 64, 0)]


@pytest.mark.parametrize("shape", EDGE, ids=["x".join(map(str, s)) for s in EDGE])
def test_edge_shapes(shape):
    M, N, K, R = shape
    _say(f"case: edge shape M={M} N={N} K={K} R={R}")
    x = synthetic.custom_inputs(M, N, K, R, seed=M * 7 + N * 13 + K + R)
    y, T = oracle_full(x)
    assert_parity(run_gpu(x), y, T, f"edge {shape}")


def test_no_write_outside_output():
    _say("case: guard band around out")
    M, N, K, R = 257, 193, 272, 32
    x = synthetic.custom_inputs(M, N, K, R, seed=77)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), 0x5A5A, dtype=torch.int16, device=DEV)
    out = buf[pad:pad + M * N].view(torch.bfloat16).view(M, N)
    got = run_gpu(x, out=out)
    host = buf.cpu().numpy().view(np.uint16)
    assert np.all(host[:pad] == 0x5A5A) and np.all(host[-pad:] == 0x5A5A)
    y, T = oracle_full(x)
    assert_parity(got, y, T, "guarded")


def test_rejects_bad_arguments_on_device():
    _say("case: C-ABI validation with real device buffers")
    x = synthetic.custom_inputs(64, 64, 128, 16, seed=1)
    d = to_device(x)
    out = torch.empty((64, 64), dtype=torch.bfloat16, device=DEV)
    base = [d[k].data_ptr() for k in ARGS] + [out.data_ptr()]
    s = torch.cuda.current_stream().cuda_stream
    assert w4.gemm_w4a4_raw(*base, 64, 64, 128, 16, s) == w4.OK
    bad = list(base)
    bad[0] += 8
    assert w4.gemm_w4a4_raw(*bad, 64, 64, 128, 16, s) == w4.EALIGN
    assert w4.gemm_w4a4_raw(*base, 64, 64, 120, 16, s) == w4.EINVAL
    bad = list(base)
    bad[8] = base[0]                       # out aliases act
    assert w4.gemm_w4a4_raw(*bad, 64, 64, 128, 16, s) == w4.EOVERLAP
    torch.cuda.synchronize()


# ---------------------------------------------------------------- fp16 variant (gemm_w4a4_f16)

def test_f16_tiny_full():
    _say("case: fp16 variant, tiny workload, every element")
    x = synthetic.make_inputs("tiny", dtype="f16")
    y, T = oracle_full(x)
    assert_parity(run_gpu(x), y, T, "f16 tiny", "f16")


@pytest.mark.parametrize("name", ["qkv", "mlp_down", "prod_k3840_n3072"])
def test_f16_workload_full_size(name):
    wl = synthetic.workload(name)
    _say(f"case: fp16 variant, {name} {wl.shape}, every element vs oracle")
    x = synthetic.make_inputs(name, dtype="f16")
    got = run_gpu(x)
    y, T = full_reference(x)
    assert_parity(got, y, T, f"f16 {name} (all {wl.M} x {wl.N})", "f16")


def test_f16_zero_main_term_shows_lora_and_bias():
    _say("case: fp16 variant, zero main term, LoRA + bias visible")
    for R in (1, 16, 32, 128):
        x = synthetic.custom_inputs(260, 200, 256, R, seed=200 + R, dtype="f16")
        x["ascales"][:] = 0
        y, T = oracle_full(x)
        got = run_gpu(x)
        assert_parity(got, y, T, f"f16 zero main R={R}", "f16")
        gv = ref.f16_bits_to_f64(got)
        assert np.all(np.abs(gv - y) <= 2 * ref.ulp_f16(y) + 1e-6)


F16_EDGE = [(1, 5, 16, 1), (7, 33, 48, 3), (257, 193, 272, 32), (300, 200, 256, 40),
            (136, 8, 32, 8), (512, 384, 1024, 0),
            # M % 8 != 0 on the fast path (act scales in 12-byte windows)
            (257, 200, 256, 32), (3, 8, 64, 8), (4095, 64, 128, 16)]


@pytest.mark.parametrize("shape", F16_EDGE, ids=["x".join(map(str, s)) for s in F16_EDGE])
def test_f16_edge_shapes(shape):
    M, N, K, R = shape
    _say(f"case: fp16 variant, edge shape M={M} N={N} K={K} R={R}")
    x = synthetic.custom_inputs(M, N, K, R, seed=M * 5 + N * 11 + K + R, dtype="f16")
    y, T = oracle_full(x)
    assert_parity(run_gpu(x), y, T, f"f16 edge {shape}", "f16")


def test_f16_overflow_becomes_infinity():
    """Columns whose value exceeds binary16's range come out as infinity, the
    others finite: every code 6 (E2M1 0x7), every scale 7.5 (0x4F), K = 64 gives
    a main term of 64 * 45 * 45 = 129600 before wcscale in [0.1, 1]."""
    _say("case: fp16 variant, outputs beyond 65504")
    M, N, K = 64, 96, 64
    x = const_inputs(M, N, K, 0, 7, 7, 0x4F, 0x4F)
    x["dtype"] = "f16"
    x["wcscale"] = np.linspace(0.1, 1.0, N).astype(np.float32)
    x["bias"] = np.zeros(N, np.float32)
    y, T = oracle_full(x)
    got = run_gpu(x)
    assert_parity(got, y, T, "f16 overflow", "f16")
    gv = ref.f16_bits_to_f64(got)
    want = ref.f16_bits_to_f64(ref.f16_rne_bits(y))
    assert np.array_equal(np.isinf(gv), np.isinf(want))
    assert np.isinf(gv).any() and np.isfinite(gv).any()


def test_f16_nan_scale_propagates():
    _say("case: fp16 variant, NaN scale byte")
    x = synthetic.custom_inputs(64, 64, 64, 8, seed=33, dtype="f16")
    x["ascales"][1, 5] = 0x7F
    got = run_gpu(x)
    y, T = oracle_full(x)
    assert_parity(got, y, T, "f16 nan scale", "f16")
    assert np.isnan(ref.f16_bits_to_f64(got)[5]).all()


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_peak_microbenchmark(kind):
    """The attainable-peak aid runs, every workgroup records its clocks, and
    its rate is positive and below the published dense peak at 2.4 GHz."""
    _say(f"case: MFMA peak microbenchmark, kind {kind}")
    clocks = torch.zeros(2 * probes.PEAK_GROUPS, dtype=torch.int64, device=DEV)
    s = torch.cuda.current_stream()
    assert probes.mfma_peak_raw(kind, 64, clocks.data_ptr(), s.cuda_stream) == w4.OK
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    assert probes.mfma_peak_raw(kind, 512, clocks.data_ptr(), s.cuda_stream) == w4.OK
    b.record()
    torch.cuda.synchronize()
    c = clocks.view(-1, 2).cpu().numpy()
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()
    mhz = np.median(c[:, 0] / (c[:, 1] / 100.0))
    assert 500 < mhz < 2600
    tf = probes.PEAK_GROUPS * 4 * 512 * 8 * probes.PEAK_FLOP[kind] / (a.elapsed_time(b) * 1e-3) / 1e12
    published = {0: 2500.0, 1: 10100.0, 2: 2500.0}[kind]
    assert 0 < tf < 1.05 * published


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_hip_graph_capture_and_replay(fmt):
    """One call captured into a HIP graph (torch.cuda.graph) replays to the
    eager result, replay after replay, with eager work and synchronisations
    in between; the launch records no memset or allocation."""
    _say(f"case: HIP graph capture and replay, {fmt}, 300x200x256 R=40")
    x = synthetic.custom_inputs(300, 200, 256, 40, seed=91, fmt=fmt)
    d = to_device(x)
    call = w4.gemm_mxfp4 if fmt == "mxfp4" else w4.gemm_w4a4
    out = torch.empty((300, 200), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
             d["lora_act_in"], d["lora_up"], out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.view(torch.int16).cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
             d["lora_act_in"], d["lora_up"], out=out)
    for rep in range(4):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), eager), rep
    a = [x[k] for k in ARGS]
    refn = ref.gemm_mxfp4_ref if fmt == "mxfp4" else ref.gemm_w4a4_ref
    tmag = ref.term_magnitude_mx if fmt == "mxfp4" else ref.term_magnitude
    assert_parity(eager.view(np.uint16), refn(*a), tmag(*a), f"graph {fmt}")


@pytest.mark.parametrize("fmt,shape", [("nvfp4", (4224, 3072, 3840, 32)), ("mxfp4", (4224, 3072, 10240, 32))])
def test_hip_graph_sliced_tail(fmt, shape):
    """A split plan whose tail runs its K in slices (three launches, float32
    sums in the output's first rows) captured into a HIP graph: every replay
    gives the eager bytes, with eager work and synchronisations in between;
    the boundary rows match the oracle."""
    M, N, K, R = shape
    p = w4.plan(M, N, K, R, fmt=fmt)
    assert p["tail_splits"] > 1
    _say(f"case: HIP graph of a K-sliced tail plan, {fmt}, {shape}")
    x = synthetic.custom_inputs(M, N, K, R, seed=92, fmt=fmt)
    d = to_device(x)
    call = w4.gemm_mxfp4 if fmt == "mxfp4" else w4.gemm_w4a4
    args = [d[k] for k in ARGS]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(*args, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.view(torch.int16).cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(*args, out=out)
    for rep in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), eager), rep
    rows = np.concatenate([np.arange(64), np.arange(p["tiles_m"] * p["block_m"] - p["block_m"], M)])
    refrows = ref.reference_rows_mx if fmt == "mxfp4" else ref.reference_rows
    y, T = refrows(x, rows)
    assert_parity(eager.view(np.uint16)[rows], y, T, f"graph sliced {fmt}")


def test_concurrent_sliced_tails():
    """Two K-sliced split plans on two streams at once, each keeping its
    float32 sums in its own output: the same bytes as one after the other."""
    M, N, K, R = 4224, 3072, 3840, 32
    assert w4.plan(M, N, K, R)["tail_splits"] > 1
    _say(f"case: two K-sliced tail plans on two streams, {M}x{N}x{K} R={R}")
    ds = [to_device(synthetic.custom_inputs(M, N, K, R, seed=s)) for s in (93, 94)]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in ds]
    for d, o in zip(ds, outs):
        w4.gemm_w4a4(*[d[k] for k in ARGS], out=o)
    torch.cuda.synchronize()
    ref_bytes = [o.clone() for o in outs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for d, o, st in zip(ds, outs, streams):
            w4.gemm_w4a4(*[d[k] for k in ARGS], out=o, stream=st)
        torch.cuda.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(outs, ref_bytes))


def test_concurrent_streams():
    """Two calls on two streams at once (different shapes, both formats)
    give the same bytes as the same calls made one after the other."""
    _say("case: concurrent calls on two streams")
    xa = synthetic.custom_inputs(1024, 768, 512, 32, seed=92)
    xb = synthetic.custom_inputs(512, 1536, 1024, 16, seed=93, fmt="mxfp4")
    da, db = to_device(xa), to_device(xb)
    oa = torch.empty((1024, 768), dtype=torch.bfloat16, device=DEV)
    ob = torch.empty((512, 1536), dtype=torch.bfloat16, device=DEV)
    args_a = [da[k] for k in ARGS]
    args_b = [db[k] for k in ARGS]
    w4.gemm_w4a4(*args_a, out=oa)
    w4.gemm_mxfp4(*args_b, out=ob)
    torch.cuda.synchronize()
    ra, rb = oa.clone(), ob.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        oa.zero_()
        ob.zero_()
        torch.cuda.synchronize()
        w4.gemm_w4a4(*args_a, out=oa, stream=s1)
        w4.gemm_mxfp4(*args_b, out=ob, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(oa, ra) and torch.equal(ob, rb)


# the 256x128 instance forced over more than one round of 128x128 tiles, with
# edges in m and n: the fast flavour (M % 8 == 0), the general one through
# M % 8 != 0, and through K % 32 != 0 (the solver may split these shapes)
TILE_256x128 = [(4320, 3064, 384, 40), (4316, 3064, 384, 40), (4300, 3000, 272, 24)]


@pytest.mark.parametrize("shape", TILE_256x128, ids=["x".join(map(str, s)) for s in TILE_256x128])
def test_256x128_instance(shape):
    M, N, K, R = shape
    v = [i for i, d in enumerate(w4.variants("nvfp4")) if (d["block_m"], d["block_n"]) == (256, 128)][0]
    _say(f"case: 256x128 instance (variant {v}), M={M} N={N} K={K} R={R}, every element")
    x = synthetic.custom_inputs(M, N, K, R, seed=M + N + K + R)
    d = to_device(x)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    rc = w4.run_raw("nvfp4", False, v, *[d[k].data_ptr() for k in ARGS], out.data_ptr(), M, N, K, R,
                    torch.cuda.current_stream().cuda_stream)
    assert rc == w4.OK, rc
    torch.cuda.synchronize()
    y, T = full_reference(x)
    assert_parity(out.view(torch.int16).cpu().numpy().view(np.uint16), y, T, f"256x128 {shape}")


# token counts that are not a multiple of 8 on the large tiles: the fast
# flavour, with the act scales read byte by byte
ODD_M = [(4095, 3072, 3072, 32), (4353, 3840, 3840, 128), (1001, 3072, 3072, 16)]


@pytest.mark.parametrize("shape", ODD_M, ids=["x".join(map(str, s)) for s in ODD_M])
def test_odd_m(shape):
    M, N, K, R = shape
    _say(f"case: M % 8 != 0 on the fast flavour, M={M} N={N} K={K} R={R}, every element")
    x = synthetic.custom_inputs(M, N, K, R, seed=M + 2 * N + K + R)
    got = run_gpu(x)
    y, T = full_reference(x)
    assert_parity(got, y, T, f"odd M {shape}")


@pytest.mark.parametrize("shift", [4, 1])
def test_misaligned_act_scales(shift):
    """Act scales at an address 4 bytes off 8-byte alignment (the fast flavour
    reads them in 12-byte windows) or at an odd address (general flavour): the
    same bytes as an aligned copy."""
    M, N, K, R = 264, 200, 256, 32
    _say(f"case: act scales at address offset {shift}, M={M} N={N} K={K} R={R}")
    x = synthetic.custom_inputs(M, N, K, R, seed=77)
    d = to_device(x)
    n = d["ascales"].numel()
    buf = torch.zeros(n + shift, dtype=torch.uint8, device=DEV)
    buf[shift:].copy_(d["ascales"].reshape(-1))
    asc = buf[shift:].view(K // 16, M)
    assert asc.data_ptr() % 8 == shift
    out_a = w4.gemm_w4a4(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
                         d["lora_act_in"], d["lora_up"])
    out_b = w4.gemm_w4a4(d["act"], asc, d["wgt"], d["wscales"], d["wcscale"], d["bias"],
                         d["lora_act_in"], d["lora_up"])
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    y, T = oracle_full(x)
    assert_parity(out_b.view(torch.int16).cpu().numpy().view(np.uint16), y, T, f"act scales at offset {shift}")


# Every compiled tile instance of both formats through gemm_w4a4_run, on the
# fast flavour (aligned), the act-scale window flavour (M % 8 != 0) and the
# general one (K % 32 != 0, R % 8 != 0), bf16 and fp16: the solver may pick
# any of them, and callers may name one. The fast and window flavours also
# with a partial last stage (K % 128 == 96: pieces past K read the next row
# or, past the tensor's end, nothing).
EVERY_VARIANT_SHAPES = [(520, 392, 640, 32), (517, 392, 640, 24), (264, 200, 272, 20), (520, 392, 608, 32),
                        (517, 392, 608, 32)]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", EVERY_VARIANT_SHAPES, ids=["x".join(map(str, s)) for s in EVERY_VARIANT_SHAPES])
def test_every_variant(shape, dtype, fmt):
    M, N, K, R = shape
    if fmt == "mxfp4" and K % 32:
        K += 16
    x = synthetic.custom_inputs(M, N, K, R, seed=M + K + R, dtype=dtype, fmt=fmt)
    x["dtype"] = dtype
    d = to_device(x)
    y, T = full_reference(x, fmt)
    half = torch.float16 if dtype == "f16" else torch.bfloat16
    for v in range(len(w4.variants(fmt))):
        p = w4.plan_variant(M, N, K, R, v, fmt=fmt)
        _say(f"case: {fmt} variant {v} ({p['block_m']}x{p['block_n']}, ring {p['stages']}, "
             f"side {p['lora_place']}), M={M} N={N} K={K} R={R} {dtype}")
        out = torch.empty((M, N), dtype=half, device=DEV)
        la = d["lora_act_in"].data_ptr() if R else 0
        lu = d["lora_up"].data_ptr() if R else 0
        rc = w4.run_raw(fmt, dtype == "f16", v, d["act"].data_ptr(), d["ascales"].data_ptr(),
                        d["wgt"].data_ptr(), d["wscales"].data_ptr(), d["wcscale"].data_ptr(),
                        d["bias"].data_ptr(), la, lu, out.data_ptr(), M, N, K, R,
                        torch.cuda.current_stream().cuda_stream)
        assert rc == w4.OK, rc
        torch.cuda.synchronize()
        assert_parity(out.view(torch.int16).cpu().numpy().view(np.uint16), y, T,
                      f"{fmt} variant {v} {shape} {dtype}", dtype)


# wcscale / bias 4 bytes off 16-byte alignment (the interface asks for 4):
# the epilogue's per-column reads, on the general flavour (K % 32 != 0) and
# on the 128x128 instance (no side region), for both operand formats.
WB_SHAPES = [(264, 200, 272, 24), (1000, 3072, 512, 16)]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("shape", WB_SHAPES, ids=["x".join(map(str, s)) for s in WB_SHAPES])
def test_wcscale_bias_4byte_aligned(shape, fmt):
    M, N, K, R = shape
    if fmt == "mxfp4" and K % 32:
        K += 16
    _say(f"case: wcscale/bias at 16-byte offset 4, {fmt}, M={M} N={N} K={K} R={R}")
    x = synthetic.custom_inputs(M, N, K, R, seed=K + R, fmt=fmt)
    d = to_device(x)
    shifted = {}
    for k in ("wcscale", "bias"):
        buf = torch.zeros(N + 1, dtype=torch.float32, device=DEV)
        buf[1:].copy_(d[k])
        shifted[k] = buf[1:]
        assert shifted[k].data_ptr() % 16 == 4
    call = w4.gemm_mxfp4 if fmt == "mxfp4" else w4.gemm_w4a4
    out_a = call(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
                 d["lora_act_in"], d["lora_up"])
    out_b = call(d["act"], d["ascales"], d["wgt"], d["wscales"], shifted["wcscale"], shifted["bias"],
                 d["lora_act_in"], d["lora_up"])
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    y, T = full_reference(x, fmt)
    assert_parity(out_b.view(torch.int16).cpu().numpy().view(np.uint16), y, T,
                  f"wcscale/bias at offset 4, {fmt} {shape}")


# Tensors just under the 2^31-byte limit the entry points accept (the kernels
# index with 32-bit offsets): the act operand (M * K/2) and the output (M * N * 2).
MAX_SHAPES = [("act", (65536, 64, 65504, 16)), ("out", (32768, 32760, 64, 8))]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("which,shape", MAX_SHAPES, ids=[w for w, _ in MAX_SHAPES])
def test_largest_tensors_sampled(which, shape, fmt):
    M, N, K, R = shape
    big = M * K // 2 if which == "act" else M * N * 2
    assert (1 << 31) - (1 << 22) < big < (1 << 31)
    _say(f"case: {which} tensor of {big} bytes, {fmt}, M={M} N={N} K={K} R={R}, sampled rows")
    x = synthetic.large_inputs(M, N, K, R, seed=95, fmt=fmt)
    d = to_device(x)
    call = w4.gemm_mxfp4 if fmt == "mxfp4" else w4.gemm_w4a4
    out = call(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
               d["lora_act_in"], d["lora_up"])
    torch.cuda.synchronize()
    rows = np.array(sorted(set([0, 1, 255, 256, M // 2, M - 257, M - 2, M - 1]) |
                           set(np.random.default_rng(13).choice(M, 24, replace=False).tolist())))
    got = out[torch.from_numpy(rows).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
    del out, d
    torch.cuda.empty_cache()
    refrows = ref.reference_rows_mx if fmt == "mxfp4" else ref.reference_rows
    y, T = refrows(x, rows)
    assert_parity(got, y, T, f"{which} max {fmt}")


# The epilogue's prefetched first LoRA chunk (side region) with R < 32: the
# ranks past R inside that chunk must be zeroed; 256x192 and 256x128 tiles,
# bf16 and fp16.
SIDE_PARTIAL = [((4096, 3072, 512, 16), "bf16"), ((4096, 3072, 512, 8), "f16"),
                ((4320, 3064, 384, 24), "f16")]


@pytest.mark.parametrize("shape,dtype", SIDE_PARTIAL,
                         ids=["x".join(map(str, s)) + "-" + d for s, d in SIDE_PARTIAL])
def test_prefetched_lora_chunk_partial_rank(shape, dtype):
    M, N, K, R = shape
    plan = w4.plan(*shape)
    assert plan["block_m"] == 256
    _say(f"case: prefetched LoRA chunk, R={R} < 32, {plan['block_m']}x{plan['block_n']}, {dtype}")
    x = synthetic.custom_inputs(M, N, K, R, seed=R + K, dtype=dtype)
    x["ascales"][:] = 0          # main term zero: the output is bias + LoRA
    got = run_gpu(x)
    y, T = full_reference(x)
    assert_parity(got, y, T, f"side chunk R={R} {dtype}", dtype)


# Split plans: the solver runs whole rounds of one instance over the first
# rows and a second launch of another over the rest (M = 4096 + 100 and
# 4096 + 257 rows at N = 3072, where 16 tile rows of 256 x 192 fill one
# round; K long enough that the second launch pays for itself): both
# launches' rows, edge tiles past M in the tail, the act-scale window flavour
# in both launches (M % 8 != 0), MXFP4 (whose tail instance takes another
# flavour than its main one at M % 4 != 0), fp16 output; tails whose K runs
# in slices (M % 8 == 0, K % 128 == 0: float32 sums in the output's first
# rows, then a reduction) with and without LoRA, and at R > 128 (LoRA in
# slice 0 over several chunks). Every element of the first 64 rows, of the
# main launch's last tile row and of every tail row.
SPLIT = [("nvfp4", "bf16", (4196, 3072, 3584, 32)), ("nvfp4", "bf16", (4353, 3072, 3840, 16)),
         ("nvfp4", "f16", (4196, 3072, 3584, 32)), ("mxfp4", "bf16", (4196, 3072, 10240, 32)),
         ("mxfp4", "bf16", (4353, 3072, 10240, 16)),
         ("nvfp4", "bf16", (4224, 3072, 3840, 32)), ("nvfp4", "f16", (4224, 3072, 3840, 32)),
         ("nvfp4", "bf16", (4352, 3072, 3840, 0)), ("nvfp4", "bf16", (4352, 3072, 2816, 136)),
         ("mxfp4", "f16", (4224, 3072, 10240, 32)), ("mxfp4", "bf16", (4352, 3072, 10240, 0))]


@pytest.mark.parametrize("fmt,dtype,shape", SPLIT, ids=[f"{f}-{d}-" + "x".join(map(str, s)) for f, d, s in SPLIT])
def test_split_plan(fmt, dtype, shape):
    M, N, K, R = shape
    p = w4.plan(M, N, K, R, fmt=fmt)
    m1 = p["tiles_m"] * p["block_m"]
    _say(f"case: {fmt} split plan M={M} N={N} K={K} R={R} {dtype}: v{p['variant']} over "
         f"{m1} rows, v{p['tail_variant']} over the last {p['tail_rows']} in {p['tail_splits']} K slices")
    assert p["tail_variant"] >= 0 and m1 + p["tail_rows"] == M
    x = synthetic.custom_inputs(M, N, K, R, seed=M + R, dtype=dtype, fmt=fmt)
    x["dtype"] = dtype
    d = to_device(x)
    half = torch.float16 if dtype == "f16" else torch.bfloat16
    fn = w4.gemm_mxfp4 if fmt == "mxfp4" else w4.gemm_w4a4
    out = fn(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
             d["lora_act_in"], d["lora_up"], dtype=half)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(64), np.arange(m1 - p["block_m"], M)])
    refrows = ref.reference_rows_mx if fmt == "mxfp4" else ref.reference_rows
    y, T = refrows(x, rows)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    assert_parity(got, y, T, f"{fmt} split {shape} {dtype}, {rows.size} rows", dtype)


# A K-sliced tail whose call does not allow slices (the output 8 bytes off
# 16-byte alignment: no float32 sums in it) runs whole, after the main
# launch; the same call on an aligned output slices. Both formats, on every
# element of the boundary rows.
@pytest.mark.parametrize("fmt,shape", [("nvfp4", (4224, 3072, 3840, 32)), ("mxfp4", (4224, 3072, 10240, 32))])
def test_sliced_tail_falls_back_on_unaligned_out(fmt, shape):
    M, N, K, R = shape
    p = w4.plan(M, N, K, R, fmt=fmt)
    assert p["tail_splits"] > 1
    x = synthetic.custom_inputs(M, N, K, R, seed=77, fmt=fmt)
    d = to_device(x)
    rows = np.concatenate([np.arange(64), np.arange(p["tiles_m"] * p["block_m"] - p["block_m"], M)])
    refrows = ref.reference_rows_mx if fmt == "mxfp4" else ref.reference_rows
    y, T = refrows(x, rows)
    for off in (0, 4):
        _say(f"case: {fmt} K-sliced tail, output offset {2 * off} bytes")
        buf = torch.empty(M * N + 8, dtype=torch.bfloat16, device=DEV)
        out = buf[off:off + M * N].view(M, N)
        rc = w4.run_raw(fmt, False, -1, *[d[k].data_ptr() for k in ARGS], out.data_ptr(), M, N, K, R,
                        torch.cuda.current_stream().cuda_stream)
        assert rc == w4.OK, rc
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
        assert_parity(got, y, T, f"{fmt} K-sliced tail, offset {2 * off}", "bf16")
