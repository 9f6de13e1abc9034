"""Parity of quantize_w4a4_act (the producer half, through the C ABI) with the
CPU oracle (oracle/quantize_ref.py). Needs a gfx950 GPU.

act and ascales are byte work: they must equal the oracle's bytes exactly.
lora_act_in is floating point: |y_gpu - y_ref| <= 4e-3 * T + 1 bf16 ulp(y_ref)
per element, T = sum_k |x * lora_down| (oracle.check_output), the same
acceptance as the fused GEMM's.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_amd as w4
import oracle.quantize_ref as qref
import oracle.w4a4_ref as ref
import synthetic

from gpu_helpers import DEV, _say, assert_parity, full_reference, to_device

pytestmark = pytest.mark.gpu


def _bits_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def run_producer(x_bits, ld_bits):
    x = _bits_dev(x_bits)
    ld = _bits_dev(ld_bits) if ld_bits.shape[0] else None
    act, asc, la = w4.quantize_w4a4_act(x, ld)
    torch.cuda.synchronize()
    la_bits = None if la is None else la.view(torch.int16).cpu().numpy().view(np.uint16)
    return act.cpu().numpy(), asc.cpu().numpy(), la_bits


def check_producer(x_bits, ld_bits, what):
    act, asc, la = run_producer(x_bits, ld_bits)
    ract, rasc = qref.quantize_nvfp4_ref(x_bits)
    bad_s = np.argwhere(asc != rasc)
    bad_a = np.argwhere(act != ract)
    _say(f"  {what}: act {act.size} bytes, ascales {asc.size} bytes, mismatches {len(bad_a)} / {len(bad_s)}")
    assert len(bad_s) == 0, ("ascales", bad_s[:8], asc[tuple(bad_s[0])], rasc[tuple(bad_s[0])])
    assert len(bad_a) == 0, ("act", bad_a[:8], act[tuple(bad_a[0])], ract[tuple(bad_a[0])])
    if ld_bits.shape[0]:
        y = qref.lora_down_ref(x_bits, ld_bits)
        T = qref.lora_down_term_magnitude(x_bits, ld_bits)
        assert_parity(la, y, T, f"{what} lora_act_in")
    else:
        assert la is None
    return act, asc, la


@pytest.mark.parametrize("name", ["tiny", "qkv", "mlp_up", "mlp_down", "ragged"])
def test_producer_workloads(name):
    wl = synthetic.workload(name)
    _say(f"case: producer at {name}'s M x K = {wl.M} x {wl.K}, R = {wl.R}")
    d = synthetic.producer_workload_inputs(name)
    check_producer(d["x"], d["lora_down"], name)


# rows not a multiple of 16 (narrow kernels) or 128 (wide kernels), K % 128
# != 0 and K % 32 == 16 (8-byte act stores), every compiled instance with R
# not a multiple of 16 or of 4 (the reduction's one-rank path): narrow for
# R <= 16, <= 32; wide with 8 rank tiles for R > 32, with 1 at R = 0 (split
# and unsplit, one and two spans a slice) and where 16-row blocks would
# overfill the chip unevenly (4352 rows), and with 2 from 4097 rows or 2^25
# elements at R <= 32; the wide kernels
# with K split (4100 rows: 33 row blocks, the last of 4 rows) and unsplit
# (257 or 258 row blocks)
EDGE = [(1, 16, 0), (17, 48, 1), (33, 144, 17), (100, 528, 32), (130, 1040, 100), (31, 2064, 128),
        (256, 128, 16), (47, 4096, 64), (64, 272, 0), (2, 16, 128), (3072, 272, 0), (3100, 400, 8),
        (4100, 4112, 100), (32800, 528, 64), (300, 3072, 33), (1000, 12288, 128),
        (4352, 1040, 9), (8200, 528, 32), (4100, 8208, 24), (33000, 272, 20), (4352, 1040, 0)]


@pytest.mark.parametrize("shape", EDGE, ids=["x".join(map(str, s)) for s in EDGE])
def test_producer_edge_shapes(shape):
    M, K, R = shape
    _say(f"case: producer edge shape M={M} K={K} R={R}")
    d = synthetic.producer_inputs(M, K, R, seed=M + K + R)
    check_producer(d["x"], d["lora_down"], f"edge {shape}")


def _bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float64), dtype=torch.float64).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_every_bf16_amax():
    """One block per positive finite bf16 value as its amax (element 0), the
    other 15 values random fractions of it: every scale decision and a wide
    spread of code decisions, byte for byte."""
    _say("case: producer, every bf16 amax as a block maximum")
    amax_bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    n = len(amax_bits)
    M, blocks = 256, -(-n // 256)
    K = 16 * blocks
    rng = np.random.default_rng(41)
    amax = ref.bf16_bits_to_f64(amax_bits)
    vals = np.zeros((M * blocks, 16))
    vals[:n, 0] = amax
    vals[:n, 1:] = amax[:, None] * rng.uniform(-1, 1, size=(n, 15))
    x = _bf16_bits(vals.reshape(M, blocks, 16).reshape(M, K))
    # keep every |x| <= amax after rounding: the maximum stays in element 0
    xv = ref.bf16_bits_to_f64(x).reshape(M * blocks, 16)
    assert np.all(np.abs(xv[:n, 1:]) <= xv[:n, :1])
    check_producer(x, np.zeros((0, K), np.uint16), "every amax")


def test_every_tie_on_every_scale():
    """Blocks whose largest value is exactly 6 s for each E4M3 value s (so the
    scale is exactly s) and whose other values are exactly the E2M1 midpoints
    t s, both signs: every tie-to-even decision of the codes, under every scale."""
    _say("case: producer, all E2M1 ties under every E4M3 scale")
    e4m3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = []
    for b in range(0x01, 0x7F):
        s = e4m3[b]
        blk = [6 * s] + [t * s for t in mids] + [-t * s for t in mids] + [-6 * s]
        rows.append(blk)
    x = _bf16_bits(np.array(rows))
    xv = ref.bf16_bits_to_f64(x)
    keep = np.all(xv == np.array(rows), axis=1)      # drop scales whose ties are not exact in bf16
    x = x[keep]
    assert keep.sum() > 100
    check_producer(x, np.zeros((0, 16), np.uint16), "ties")


def test_special_values():
    _say("case: producer, zeros, signed zeros, NaN / inf blocks, saturation, tiny scales")
    v = np.zeros((8, 64))
    v[1, :16] = -0.0
    v[2, 5] = np.nan
    v[3, 17] = np.inf
    v[3, 40] = -np.inf
    v[4, :] = 3.0e38
    v[5, :16] = np.linspace(-1e-5, 1e-5, 16)
    v[6, :] = np.tile([1e-3, -2e-3, 5e-4, 0.0], 16)
    v[7, :] = np.tile([448 * 6, -1.0, 0.5, 2688.0], 16)
    check_producer(_bf16_bits(v), np.zeros((0, 64), np.uint16), "special values")


def test_producer_guard_band():
    """Nothing outside act, ascales and lora_act_in is written."""
    M, K, R = 37, 272, 24
    _say(f"case: producer guard band M={M} K={K} R={R}")
    d = synthetic.producer_inputs(M, K, R, seed=77)
    x, ld = _bits_dev(d["x"]), _bits_dev(d["lora_down"])
    pad = 256
    bufs = {}
    for name, n, dt in (("act", M * K // 2, torch.uint8), ("ascales", K // 16 * M, torch.uint8),
                        ("la", M * R, torch.int16)):
        b = torch.full((n + 2 * pad,), 0x5A, dtype=dt, device=DEV)
        bufs[name] = b
    act = bufs["act"][pad:pad + M * K // 2].view(M, K // 2)
    asc = bufs["ascales"][pad:pad + K // 16 * M].view(K // 16, M)
    la = bufs["la"][pad:pad + M * R].view(M, R).view(torch.bfloat16)
    w4.quantize_w4a4_act(x, ld, act, asc, la)
    torch.cuda.synchronize()
    for name, b in bufs.items():
        h = b.cpu().numpy()
        assert np.all(h[:pad] == 0x5A) and np.all(h[-pad:] == 0x5A), name
    ract, rasc = qref.quantize_nvfp4_ref(d["x"])
    assert np.array_equal(act.cpu().numpy(), ract) and np.array_equal(asc.cpu().numpy(), rasc)


def test_deterministic():
    d = synthetic.producer_inputs(300, 1024, 64, seed=78)
    a = run_producer(d["x"], d["lora_down"])
    b = run_producer(d["x"], d["lora_down"])
    assert all(np.array_equal(p, q) for p, q in zip(a, b))


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_layer_end_to_end(name):
    """The whole W4A4 layer on the GPU: x -> quantize_w4a4_act -> gemm_w4a4,
    against the oracle of each half chained the same way (the GEMM oracle
    takes the act / ascales the quantiser oracle produced, which the GPU's
    equal byte for byte, and the GPU's lora_act_in, checked above)."""
    wl = synthetic.workload(name)
    M, N, K, R = wl.shape
    _say(f"case: layer end to end at {name} {wl.shape}")
    d = synthetic.producer_workload_inputs(name)
    g = synthetic.make_inputs(name)
    x, ld = _bits_dev(d["x"]), _bits_dev(d["lora_down"])
    act, asc, la = w4.quantize_w4a4_act(x, ld)
    dev = to_device(g)
    out = w4.gemm_w4a4(act, asc, dev["wgt"], dev["wscales"], dev["wcscale"], dev["bias"], la, dev["lora_up"])
    torch.cuda.synchronize()
    ract, rasc = qref.quantize_nvfp4_ref(d["x"])
    assert np.array_equal(act.cpu().numpy(), ract) and np.array_equal(asc.cpu().numpy(), rasc)
    chain = dict(g, act=ract, ascales=rasc,
                 lora_act_in=la.view(torch.int16).cpu().numpy().view(np.uint16))
    y, T = full_reference(chain)
    assert_parity(out.view(torch.int16).cpu().numpy().view(np.uint16), y, T, f"layer {name}")


def test_split_calls_of_different_sizes():
    """Consecutive calls whose K is split over workgroups (few row blocks, many
    spans), with different numbers of row blocks and ranks: the arrival
    counters live in the same scratch bytes in every call and must be back at
    zero after each."""
    for shape in [(1000, 8192, 16), (2000, 4096, 8), (33, 4160, 17), (4160, 4096, 128), (2000, 4096, 8),
                  (200, 2048, 128), (4100, 4112, 100), (1000, 8192, 16)]:
        M, K, R = shape
        _say(f"case: producer split sequence M={M} K={K} R={R}")
        d = synthetic.producer_inputs(M, K, R, seed=M * 7 + K + R)
        check_producer(d["x"], d["lora_down"], f"sequence {shape}")


def test_split_calls_on_two_streams_overlap_safely():
    """Split calls on two streams, enqueued alternately with no ordering
    between the streams: each stream has its own scratch (counters and
    partial sums), so both results equal those of the same calls made one
    after another."""
    shapes = [(1000, 8192, 16), (2000, 4096, 8)]   # both split K (narrow kernels, arrival counters)
    dev = torch.device("cuda:0")
    bufs = []
    for M, K, R in shapes:
        d = synthetic.producer_inputs(M, K, R, seed=M * 5 + K + R)
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
        ld = torch.from_numpy(d["lora_down"].view(np.int16)).view(torch.bfloat16).to(dev)
        bufs.append((x, ld, w4.quantize_w4a4_act(x, ld)))
    torch.cuda.synchronize()
    want = [tuple(t.clone() for t in b[2]) for b in bufs]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    for _ in range(20):
        for (x, ld, outs), s in zip(bufs, streams):
            act, asc, la = outs
            M, K = x.shape
            rc = w4.quantize_raw(x.data_ptr(), ld.data_ptr(), act.data_ptr(), asc.data_ptr(), la.data_ptr(),
                                 M, K, ld.shape[0], s.cuda_stream)
            assert rc == w4.OK, w4.strerror(rc)
    torch.cuda.synchronize()
    for (x, ld, outs), w, shape in zip(bufs, want, shapes):
        _say(f"case: producer on two streams {shape}")
        for got, exp in zip(outs, w):
            assert torch.equal(got, exp), shape


def test_plan_on_the_device_matches_the_host_model():
    """On the GPU the planner reads the device's compute-unit count (256 on
    MI355X): the choices pinned on the CPU (tests/test_producer_plan.py, which
    assume 256) hold here too."""
    import torch as _t
    cus = _t.cuda.get_device_properties(0).multi_processor_count
    _say(f"case: producer plan on the device ({cus} compute units)")
    if cus != 256:
        pytest.skip(f"{cus} compute units: the pinned plans assume 256")
    assert w4.quantize_plan(4096, 12288, 128)["k_slices"] == 8
    assert w4.quantize_plan(1000, 3072, 16)["k_slices"] == 3
    assert w4.quantize_plan(4352, 10240, 32)["variant"] == 4
