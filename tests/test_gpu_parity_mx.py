"""Parity of the MXFP4 entry points (gemm_mxfp4, gemm_mxfp4_f16) with the CPU
oracle (oracle.gemm_mxfp4_ref). Needs a gfx950 GPU.

Same acceptance as the NVFP4 path: |y_gpu - y_ref| <= 4e-3 * T + 1 ulp(y_ref)
of the output type, T = |wcscale| sum_k |A W| + |bias| + sum_r |la lu|.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_amd as w4
import oracle.w4a4_ref as ref
import synthetic

from gpu_helpers import ARGS, DEV, _say, assert_parity, full_reference, to_device

pytestmark = pytest.mark.gpu


def run_mx(x, out=None):
    d = to_device(x)
    half = torch.float16 if x.get("dtype", "bf16") == "f16" else torch.bfloat16
    o = w4.gemm_mxfp4(d["act"], d["ascales"], d["wgt"], d["wscales"], d["wcscale"], d["bias"],
                      d["lora_act_in"], d["lora_up"], out=out, dtype=half)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_mx(x):
    a = [x[k] for k in ARGS]
    dt = x.get("dtype", "bf16")
    return ref.gemm_mxfp4_ref(*a, dtype=dt), ref.term_magnitude_mx(*a, dtype=dt)


def mx_inputs(M, N, K, R, seed, dtype="bf16", **kw):
    return synthetic.custom_inputs(M, N, K, R, seed=seed, dtype=dtype, fmt="mxfp4", **kw)


# ---------------------------------------------------------------- workloads

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mx_tiny_full(dtype):
    _say(f"case: MXFP4 tiny workload 256x256x512 R=32 ({dtype}), every element")
    x = synthetic.make_inputs("tiny", dtype=dtype, fmt="mxfp4")
    y, T = oracle_mx(x)
    assert_parity(run_mx(x), y, T, f"mx tiny {dtype}", dtype)


@pytest.mark.parametrize("name", ["qkv", "mlp_up", "mlp_down", "ragged", "prod_k3840_n3072",
                                  "prod_k15360_n3840"])
def test_mx_workload_full_size(name):
    wl = synthetic.workload(name)
    _say(f"case: MXFP4 {name} {wl.shape}, full-size launch, every element vs oracle")
    x = synthetic.make_inputs(name, fmt="mxfp4")
    got = run_mx(x)
    y, T = full_reference(x, "mxfp4")
    assert_parity(got, y, T, f"mx {name} (all {wl.M} x {wl.N})")
    vals = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(vals).all()


def test_mx_ceiling_mode_full_size():
    _say("case: MXFP4 qkv ceiling mode (no LoRA, no affine), every element vs oracle")
    x = synthetic.no_lora_affine(synthetic.make_inputs("qkv", fmt="mxfp4"))
    got = run_mx(x)
    y, T = full_reference(x, "mxfp4")
    assert_parity(got, y, T, "mx qkv ceiling")


def test_mx_f16_full_size():
    wl = synthetic.workload("mlp_down")
    _say(f"case: MXFP4 fp16 variant, mlp_down {wl.shape}, every element")
    x = synthetic.make_inputs("mlp_down", dtype="f16", fmt="mxfp4")
    got = run_mx(x)
    y, T = full_reference(x, "mxfp4")
    assert_parity(got, y, T, "mx f16 mlp_down", "f16")


def test_mx_deterministic_bytes():
    _say("case: MXFP4 determinism, ragged workload twice")
    x = synthetic.make_inputs("ragged", fmt="mxfp4")
    assert np.array_equal(run_mx(x), run_mx(x))


# ---------------------------------------------------------------- exhaustive scales

def _mx_decode_case(side):
    """Every (E2M1 code, UE8M0 byte) pair on one operand side, K = 32 (one
    block). The other side is code 1.0 with scale 2^-5, so each output is the
    sum of 32 equal products v * 2^(b-127) * 2^-5 = v * 2^(b-127), and no
    partial sum is larger than the result."""
    rows = 16 * 256
    code = np.arange(rows) % 16
    sbyte = (np.arange(rows) // 16).astype(np.uint8)
    packed = (code | (code << 4)).astype(np.uint8)[:, None].repeat(16, axis=1)
    other = 64
    one_packed = np.full((other, 16), 0x22, np.uint8)          # E2M1 1.0
    one_scale = np.full((1, other), 127 - 5, np.uint8)          # 2^-5
    x = dict(K=32, R=0)
    if side == "act":
        x.update(M=rows, N=other, act=packed, ascales=sbyte[None, :], wgt=one_packed,
                 wscales=one_scale)
    else:
        x.update(M=other, N=rows, act=one_packed, ascales=one_scale, wgt=packed,
                 wscales=sbyte[None, :])
    x["wcscale"] = np.ones(x["N"], np.float32)
    x["bias"] = np.zeros(x["N"], np.float32)
    x["lora_act_in"] = np.zeros((x["M"], 0), np.uint16)
    x["lora_up"] = np.zeros((0, x["N"]), np.uint16)
    return x, sbyte


@pytest.mark.parametrize("side", ["act", "wgt"])
def test_mx_scale_exhaustive(side):
    """Exact, value for value, wherever every product and partial sum is a
    normal fp32 number (scale bytes 8 .. 250); NaN for byte 255; within the
    tolerance (or flushed below 2^-126) at the subnormal end."""
    _say(f"case: MXFP4 exhaustive scale bytes, {side} side, 16 codes x 256 bytes")
    x, sbyte = _mx_decode_case(side)
    got = run_mx(x)
    y, T = oracle_mx(x)
    gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    byte = sbyte[:, None] if side == "act" else sbyte[None, :]
    byte = np.broadcast_to(byte, y.shape)
    nan_y = np.isnan(y)
    assert np.array_equal(nan_y, byte == 255)
    assert np.array_equal(np.isnan(gv), nan_y)
    normal = (byte >= 8) & (byte <= 250)
    assert np.array_equal(gv[normal], y[normal])
    # everything above the subnormal end, overflow to infinity included
    sel = sbyte >= 8
    pick = (lambda a: a[sel]) if side == "act" else (lambda a: a[:, sel])
    assert_parity(pick(got), pick(y), pick(T), "mx scale bytes >= 8")
    low = byte < 8
    bound = np.maximum(ref.tolerance_bound(y, T), 2.0 ** -126)
    assert np.all(np.abs(gv[low] - y[low]) <= bound[low])


# ---------------------------------------------------------------- structured probes

def test_mx_probe_nibble_and_scale_layout():
    """One nonzero nibble (or one odd scale byte) at a time: a wrong nibble
    order, k-block or scale row shows up as a wrong value at a known place."""
    _say("case: MXFP4 single-nibble and single-scale probes")
    rng = np.random.default_rng(4)
    M, N, K = 132, 200, 384
    for k0 in (0, 31, 32, 127, 128, 200, 383):
        x = mx_inputs(M, N, K, 0, seed=41)
        x["act"][:] = 0
        x["act"][33, k0 // 2] = np.uint8(13 << (4 * (k0 % 2)))
        x["wgt"][:] = np.uint8(4 | (2 << 4))
        x["wscales"] = (127 + rng.integers(-2, 3, size=x["wscales"].shape)).astype(np.uint8)
        y, T = oracle_mx(x)
        got = run_mx(x)
        assert_parity(got, y, T, f"mx nibble k0={k0}")
    for (kb0, m0, kb1, n1) in [(1, 3, 4, 2), (2, 130, 2, 190), (11, 131, 0, 0), (5, 64, 7, 199)]:
        x = mx_inputs(M, N, K, 0, seed=42)
        x["act"][:] = np.uint8(2 | (2 << 4))
        x["wgt"][:] = np.uint8(2 | (2 << 4))
        x["ascales"][:] = 127
        x["wscales"][:] = 127
        x["ascales"][kb0, m0] = 130
        x["wscales"][kb1, n1] = 124
        y, T = oracle_mx(x)
        got = run_mx(x)
        assert_parity(got, y, T, f"mx scale probe {(kb0, m0, kb1, n1)}")
        gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(gv, ref.bf16_bits_to_f64(ref.bf16_rne_bits(y)))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mx_zero_main_term_shows_lora_and_bias(dtype):
    """Act codes all zero: y = bias + LoRA exactly as far as
    fp32 holds it, so a dropped or mis-scaled LoRA or bias term fails."""
    _say(f"case: MXFP4 zero main term ({dtype}), LoRA + bias visible")
    ulp = ref.ulp_bf16 if dtype == "bf16" else ref.ulp_f16
    for R in (1, 16, 32, 128):
        x = mx_inputs(260, 200, 256, R, seed=300 + R, dtype=dtype)
        x["act"][:] = 0
        y, T = oracle_mx(x)
        got = run_mx(x)
        assert_parity(got, y, T, f"mx zero main R={R}", dtype)
        gv = ref.half_bits_to_f64(got, dtype)
        assert np.all(np.abs(gv - y) <= 2 * ulp(y) + 1e-6)


@pytest.mark.parametrize("shape", [(256, 200, 256, 160), (256, 192, 128, 1024), (260, 200, 256, 1000),
                                   (4096, 3072, 128, 160), (4096, 3072, 128, 1024)],
                         ids=["fast_R160", "fast_R1024", "general_R1000", "256x192_R160", "256x192_R1024"])
def test_mx_probe_large_rank_lora_visible(shape):
    """As the NVFP4 probe: act codes zero, y = bias + a sum of R LoRA
    products, ranks far past the pages' 128."""
    M, N, K, R = shape
    _say(f"case: MXFP4 zero main term at R={R}, M={M} N={N} K={K}")
    x = mx_inputs(M, N, K, R, seed=600 + R)
    x["act"][:] = 0
    y, T = oracle_mx(x)
    got = run_mx(x)
    assert_parity(got, y, T, f"mx zero main R={R}")
    gv = ref.half_bits_to_f64(got, "bf16")
    assert np.all(np.abs(gv - y) <= 2 * ref.ulp_bf16(y) + 1e-5)


def test_mx_nan_scale_propagates():
    _say("case: MXFP4 NaN scale byte (0xFF)")
    x = mx_inputs(64, 64, 128, 0, seed=51)
    x["ascales"][1, 5] = 0xFF
    x["wscales"][3, 9] = 0xFF
    got = run_mx(x)
    y, T = oracle_mx(x)
    assert_parity(got, y, T, "mx nan scale")
    gv = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.isnan(gv[5]).all() and np.isnan(gv[:, 9]).all()
    assert np.isfinite(np.delete(np.delete(gv, 5, 0), 9, 1)).all()


# ---------------------------------------------------------------- edge shapes

MX_EDGE = [
    # general flavour: K % 128 != 0, M % 4 != 0, N % 8 != 0 or R % 8 != 0
    (1, 1, 32, 0), (1, 5, 32, 1), (7, 33, 96, 3), (33, 200, 160, 16), (257, 193, 288, 32),
    (300, 129, 224, 17), (129, 1, 64, 8), (2, 1000, 352, 24), (1000, 64, 416, 40),
    (64, 64, 4096, 128),
    # fast flavour (K % 128 == 0, M % 4 == 0, N % 8 == 0, R % 8 == 0): edge
    # tiles in m and n, several LoRA chunks, the last one partly inside R
    (300, 200, 256, 40), (104, 3000, 512, 72), (136, 8, 128, 8), (64, 64, 384, 24),
    (260, 200, 640, 16), (512, 384, 1024, 0), (4, 8, 128, 0)]


@pytest.mark.parametrize("shape", MX_EDGE, ids=["x".join(map(str, s)) for s in MX_EDGE])
def test_mx_edge_shapes(shape):
    M, N, K, R = shape
    _say(f"case: MXFP4 edge shape M={M} N={N} K={K} R={R}")
    x = mx_inputs(M, N, K, R, seed=M * 3 + N * 17 + K + R)
    y, T = oracle_mx(x)
    assert_parity(run_mx(x), y, T, f"mx edge {shape}")


@pytest.mark.parametrize("shape", [(7, 33, 96, 3), (300, 200, 256, 40), (136, 8, 128, 8)])
def test_mx_f16_edge_shapes(shape):
    M, N, K, R = shape
    _say(f"case: MXFP4 fp16 edge shape M={M} N={N} K={K} R={R}")
    x = mx_inputs(M, N, K, R, seed=M * 5 + N * 19 + K + R, dtype="f16")
    y, T = oracle_mx(x)
    assert_parity(run_mx(x), y, T, f"mx f16 edge {shape}", "f16")


def test_mx_no_write_outside_output():
    _say("case: MXFP4 guard band around out")
    M, N, K, R = 257, 193, 288, 32
    x = mx_inputs(M, N, K, R, seed=78)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), 0x5A5A, dtype=torch.int16, device=DEV)
    out = buf[pad:pad + M * N].view(torch.bfloat16).view(M, N)
    got = run_mx(x, out=out)
    host = buf.cpu().numpy().view(np.uint16)
    assert np.all(host[:pad] == 0x5A5A) and np.all(host[-pad:] == 0x5A5A)
    y, T = oracle_mx(x)
    assert_parity(got, y, T, "mx guarded")


def test_mx_rejects_bad_arguments_on_device():
    _say("case: MXFP4 C-ABI validation with real device buffers")
    x = mx_inputs(64, 64, 128, 16, seed=2)
    d = to_device(x)
    out = torch.empty((64, 64), dtype=torch.bfloat16, device=DEV)
    base = [d[k].data_ptr() for k in ARGS] + [out.data_ptr()]
    s = torch.cuda.current_stream().cuda_stream
    assert w4.gemm_mxfp4_raw(*base, 64, 64, 128, 16, s) == w4.OK
    bad = list(base)
    bad[0] += 8
    assert w4.gemm_mxfp4_raw(*bad, 64, 64, 128, 16, s) == w4.EALIGN
    assert w4.gemm_mxfp4_raw(*base, 64, 64, 112, 16, s) == w4.EINVAL
    bad = list(base)
    bad[8] = base[0]
    assert w4.gemm_mxfp4_raw(*bad, 64, 64, 128, 16, s) == w4.EOVERLAP
    torch.cuda.synchronize()



@pytest.mark.parametrize("shape,dtype", [((4096, 3072, 512, 16), "bf16"), ((4096, 3072, 512, 8), "f16")])
def test_mx_prefetched_lora_chunk_partial_rank(shape, dtype):
    """The first LoRA chunk prefetched into LDS (act rows and lora_up rows)
    with R < 32: ranks past R must contribute nothing."""
    M, N, K, R = shape
    plan = w4.plan(*shape, fmt="mxfp4")
    assert (plan["block_m"], plan["block_n"]) == (256, 192)
    _say(f"case: MXFP4 prefetched LoRA chunk, R={R} < 32, {dtype}")
    x = mx_inputs(M, N, K, R, seed=R + K + 1, dtype=dtype)
    x["act"][:] = 0              # main term zero: the output is bias + LoRA
    got = run_mx(x)
    y, T = full_reference(x, "mxfp4")
    assert_parity(got, y, T, f"mx side chunk R={R} {dtype}", dtype)


MX_ODD_M = [((4095, 3072, 3072, 32), "bf16"), ((4093, 3072, 512, 16), "bf16"),
            ((4353, 3840, 3840, 128), "bf16"), ((4095, 3072, 512, 8), "f16")]


@pytest.mark.parametrize("shape,dtype", MX_ODD_M, ids=["x".join(map(str, s)) + "-" + d for s, d in MX_ODD_M])
def test_mx_odd_m_act_scale_windows(shape, dtype):
    """M % 4 != 0 on the 256x192 tile: the fast flavour reads each k-block row
    of act scales through a 4-byte aligned window (the last one clamped to
    the tensor's end), every row offset into it different."""
    M, N, K, R = shape
    plan = w4.plan(*shape, fmt="mxfp4")
    assert (plan["block_m"], plan["block_n"]) == (256, 192)
    _say(f"case: MXFP4 odd M with act-scale windows {shape} {dtype}")
    x = mx_inputs(M, N, K, R, seed=M + K + R, dtype=dtype)
    got = run_mx(x)
    y, T = full_reference(x, "mxfp4")
    assert_parity(got, y, T, f"mx odd M {shape} {dtype}", dtype)
