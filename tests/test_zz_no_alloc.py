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
