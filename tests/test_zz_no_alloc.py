"""quantize_w4a4_act_noalloc, the entry point that allocates nothing (its
split-K scratch is a fixed device array per GPU), against quantize_w4a4_act
through the C ABI: calls in a row whose K is split over workgroups, so
that the scratch is used, each pair's second on a smaller input (narrow
kernels with arrival counters, then the wide kernel with its reduction
launch, whose partial sums are larger than the first pair's). act, ascales and
lora_act_in must equal quantize_w4a4_act's bit for bit (same kernels, same
order of additions), and meet the oracle's bar (byte-exact act / ascales,
lora_act_in within 4e-3 T + 1 ulp). Needs a gfx950 GPU."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_amd as w4
import oracle.quantize_ref as qref
import synthetic

from gpu_helpers import DEV, _say, assert_parity

pytestmark = pytest.mark.gpu


def _bits_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def _run(entry, x, ld, M, K, R):
    # outputs pre-filled with a pattern no call writes everywhere by chance
    act = torch.full((M, K // 2), 0xA5, dtype=torch.uint8, device=DEV)
    asc = torch.full((K // 16, M), 0xA5, dtype=torch.uint8, device=DEV)
    la = torch.full((M, R), 0x7FC1, dtype=torch.int16, device=DEV)
    stream = torch.cuda.current_stream()
    rc = getattr(w4, entry)(x.data_ptr(), ld.data_ptr(), act.data_ptr(), asc.data_ptr(), la.data_ptr(),
                            M, K, R, stream.cuda_stream)
    assert rc == w4.OK, (entry, rc, w4.strerror(rc))
    torch.cuda.synchronize()
    return act.cpu().numpy(), asc.cpu().numpy(), la.cpu().numpy().view(np.uint16)


def test_noalloc_matches_quantize_w4a4_act():
    for M, K, R in [(1000, 8192, 32), (200, 4096, 16), (4160, 4096, 128), (300, 2048, 64)]:
        _say(f"case: no-allocation entry point M={M} K={K} R={R}")
        d = synthetic.producer_inputs(M, K, R, seed=M + 3 * K + R)
        x, ld = _bits_dev(d["x"]), _bits_dev(d["lora_down"])
        want = _run("quantize_raw", x, ld, M, K, R)
        got = _run("quantize_noalloc_raw", x, ld, M, K, R)
        for name, a, b in zip(("act", "ascales", "lora_act_in"), got, want):
            assert np.array_equal(a, b), (name, np.argwhere(a != b)[:4])
        ract, rasc = qref.quantize_nvfp4_ref(d["x"])
        assert np.array_equal(got[0], ract) and np.array_equal(got[1], rasc)
        assert_parity(got[2], qref.lora_down_ref(d["x"], d["lora_down"]),
                      qref.lora_down_term_magnitude(d["x"], d["lora_down"]), f"no-alloc {M}x{K}x{R}")


def test_noalloc_captures_into_a_hip_graph():
    """The entry point's purpose: it can be captured (nothing is allocated,
    no memset is recorded: the split's counters are returned to zero by the
    kernels themselves). A narrow split (arrival counters) and a wide split
    (reduction launch) are each captured into a HIP graph and replayed four
    times with eager work and synchronisations in between; every replay
    equals the eager call."""
    for M, K, R in [(1000, 8192, 32), (4160, 4096, 128)]:
        _say(f"case: no-allocation entry point under graph capture M={M} K={K} R={R}")
        d = synthetic.producer_inputs(M, K, R, seed=M + 5 * K + R)
        x, ld = _bits_dev(d["x"]), _bits_dev(d["lora_down"])
        want = _run("quantize_noalloc_raw", x, ld, M, K, R)
        act = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
        asc = torch.empty((K // 16, M), dtype=torch.uint8, device=DEV)
        la = torch.empty((M, R), dtype=torch.int16, device=DEV)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rc = w4.quantize_noalloc_raw(x.data_ptr(), ld.data_ptr(), act.data_ptr(), asc.data_ptr(), la.data_ptr(),
                                         M, K, R, torch.cuda.current_stream().cuda_stream)
            assert rc == w4.OK, w4.strerror(rc)
        for rep in range(4):
            for t in (act, asc, la):
                t.fill_(0x5A)
            _run("quantize_noalloc_raw", x, ld, 33, 4096, 17)   # eager split call in between (same scratch)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (act.cpu().numpy(), asc.cpu().numpy(), la.cpu().numpy().view(np.uint16))
            for name, a, b in zip(("act", "ascales", "lora_act_in"), got, want):
                assert np.array_equal(a, b), (name, rep)
