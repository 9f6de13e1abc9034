"""Host-side rules of split plans (no GPU): where the solver runs a second
launch over the last rows, when that launch runs its K in slices, and the
bounds the slices' float32 sums must keep inside the output."""
import itertools

import pytest

import bit_quantized_gemm_amd as w4

SHAPES = [(M, N, K, R) for M, N, K, R in itertools.product(
    (1000, 2000, 4096, 4196, 4224, 4352, 4353, 8192 + 256), (3072, 3840, 15360), (256, 3072, 3840, 10240), (0, 32, 128))]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_split_plan_invariants(fmt):
    seen_split = seen_sliced = 0
    for M, N, K, R in SHAPES:
        p = w4.plan(M, N, K, R, fmt=fmt)
        if p["tail_variant"] < 0:
            assert p["tail_rows"] == 0 and p["tail_splits"] == 1
            assert p["tiles_m"] * p["block_m"] >= M
            continue
        seen_split += 1
        m1 = p["tiles_m"] * p["block_m"]
        assert 0 < p["tail_rows"] < M and m1 + p["tail_rows"] == M        # whole main tile rows, the rest in the tail
        assert p["block_m"] % p["tail_block_m"] == 0                     # the tail's first tile row is whole
        S = p["tail_splits"]
        tiles = -(-p["tail_rows"] // p["tail_block_m"]) * -(-N // p["tail_block_n"])
        assert p["tail_grid"] == tiles * S
        if S > 1:
            seen_sliced += 1
            assert 2 <= S <= 8
            assert S * p["tail_rows"] * 4 <= m1 * 2                      # float32 sums fit in the main rows
            assert K % 128 == 0 and N % 8 == 0 and (R == 0 or R % 8 == 0)
            assert M % (8 if fmt == "nvfp4" else 4) == 0
            assert K // 128 >= 2 * S                                     # at least two stages a slice
            assert p["tail_grid"] <= 256 * (2 if fmt == "mxfp4" else 1)  # one round of sliced workgroups
    assert seen_split > 0 and seen_sliced > 0


def test_short_k_never_splits():
    """A second launch costs a fixed share; at two stages it never pays."""
    for M, N in ((4352, 3072), (4196, 3072), (4224, 3072)):
        for fmt in ("nvfp4", "mxfp4"):
            assert w4.plan(M, N, 256, 32, fmt=fmt)["tail_variant"] == -1


def test_production_shape_plans():
    """The pages' M = 4352 shapes: the 17th tile row of 256 x 192 tiles as a
    K-sliced 64 x 192 tail where the tail is one tile row (NVFP4), and whole
    plans where no split pays."""
    p = w4.plan(4352, 3072, 3840, 128)
    assert (p["block_m"], p["block_n"], p["tiles_m"]) == (256, 192, 16)
    assert (p["tail_block_m"], p["tail_rows"], p["tail_splits"]) == (64, 256, 4)
    assert w4.plan(4352, 3072, 10240, 32)["tail_splits"] == 4
    assert w4.plan(4352, 3072, 10240, 32, fmt="mxfp4")["tail_splits"] == 8
    assert w4.plan(4352, 3840, 15360, 128)["tail_variant"] == -1
    assert w4.plan(4096, 3072, 3072, 32)["tail_variant"] == -1               # the headline shape: one launch


def test_no_slices_without_the_fast_flavour():
    """M % 8 != 0 (NVFP4's byte-wise act scales) or K % 128 != 0 keep the
    tail whole."""
    assert w4.plan(4353, 3072, 3840, 128)["tail_splits"] == 1
    assert w4.plan(4356, 3072, 3840, 128)["tail_splits"] == 1
    p = w4.plan(4352, 3072, 3840 + 64, 128)
    assert p["tail_splits"] == 1


def test_forced_instance_never_splits():
    for v in range(len(w4.variants("nvfp4"))):
        p = w4.plan_variant(4352, 3072, 3840, 128, v)
        assert p["tail_variant"] == -1 and p["tail_splits"] == 1
