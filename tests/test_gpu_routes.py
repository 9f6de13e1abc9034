"""The two ways of running NVFP4's block-scaled product on gfx950's matrix
cores (measurement aids, not the operator): the scaled-FP4-MFMA route's
one-tile kernel against the float64 reference, and both per-block rate cores
on every SIMD. The route gemm_w4a4 takes is covered by the parity suites."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_amd as w4
from bit_quantized_gemm_amd import probes
import oracle.w4a4_ref as ref

from gpu_helpers import DEV, _say

pytestmark = pytest.mark.gpu


def tile_inputs(K: int, seed: int):
    """Random packed codes (all 16 E2M1 codes on both operands) and positive
    E4M3 scales over the whole finite range, zero and subnormals included."""
    rng = np.random.default_rng(seed)
    act = rng.integers(0, 256, size=(32, K // 2), dtype=np.uint8)
    wgt = rng.integers(0, 256, size=(32, K // 2), dtype=np.uint8)
    asc = rng.integers(0, 0x7F, size=(K // 16, 32), dtype=np.uint8)
    wsc = rng.integers(0, 0x7F, size=(K // 16, 32), dtype=np.uint8)
    return act, asc, wgt, wsc


@pytest.mark.parametrize("K,seed", [(16, 1), (64, 2), (1024, 3), (3072, 4)])
def test_route_b_tile_matches_the_reference(K, seed):
    """Each block's partial sum is exact (16 E2M1 products) and so is its
    product with the two block scales; only the fp32 accumulation over the
    K/16 blocks rounds, at most half an ulp of the running sum per block."""
    _say(f"case: route B tile, K={K} seed={seed}")
    act, asc, wgt, wsc = tile_inputs(K, seed)
    S = ref.main_product(act, asc, wgt, wsc)
    mag = np.abs(ref.dequantize(act, asc)) @ np.abs(ref.dequantize(wgt, wsc)).T
    d = [torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (act, asc, wgt, wsc)]
    out = torch.full((32, 32), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream()
    assert probes.route_b_tile_raw(*(v.data_ptr() for v in d), out.data_ptr(), K, s.cuda_stream) == w4.OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    bound = (K // 16) * 2.0 ** -24 * mag
    err = np.abs(got - S)
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))


def test_route_b_tile_single_block_is_bit_exact():
    """One block: nothing rounds at all."""
    _say("case: route B tile, one block")
    act, asc, wgt, wsc = tile_inputs(16, 7)
    S = ref.main_product(act, asc, wgt, wsc)
    d = [torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (act, asc, wgt, wsc)]
    out = torch.empty((32, 32), dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream()
    assert probes.route_b_tile_raw(*(v.data_ptr() for v in d), out.data_ptr(), 16, s.cuda_stream) == w4.OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), S)


@pytest.mark.parametrize("route", [0, 1])
def test_route_core_runs_on_every_simd(route):
    _say(f"case: route core {route}")
    clocks = torch.zeros(2 * probes.PEAK_GROUPS, dtype=torch.int64, device=DEV)
    s = torch.cuda.current_stream()
    assert probes.route_core_raw(route, 192, clocks.data_ptr(), s.cuda_stream) == w4.OK
    torch.cuda.synchronize()
    c = clocks.view(-1, 2).cpu().numpy()
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()
    # at least the 12 MFMAs of a block (each occupies the matrix core for
    # 8 or more cycles) per block and wave
    assert np.median(c[:, 0]) / 192 >= 12 * 8
