"""The producer's launch plan (quantize_w4a4_act_plan, host only; CPU).

The instance and K split follow measurements on MI355X (the kernel source's
notes): narrow kernels at 0 < R <= 32 unless their 16-row blocks overfill
the compute units unevenly or, at R > 16, from 4097 rows or 2^25 elements;
the wide kernel with one rank tile at R = 0 and with 8 above R = 32; K split so that every row block's
workgroups fit one round on the compute units (256 here: no device is
current on the CPU, and MI355X has 256). These tests pin those decisions and
the plan's own consistency."""
import itertools

import pytest

import bit_quantized_gemm_amd as w4

NOALLOC = 4096 + (16 << 20)


@pytest.mark.parametrize("shape,variant,wide,rank_tiles,k_slices,launches", [
    ((4096, 3072, 32), 1, 0, 2, 1, 1),      # qkv: narrow, 256 row blocks fill the chip
    ((4096, 3072, 16), 0, 0, 1, 1, 1),
    ((4096, 3072, 0), 3, 1, 1, 8, 1),       # no LoRA: the wide kernel, no partial sums
    ((1000, 3072, 16), 0, 0, 1, 3, 1),      # ragged: narrow, one span per wave
    ((4096, 12288, 128), 2, 1, 8, 8, 2),    # mlp_down: wide, reduction launch
    ((4096, 12288, 32), 4, 1, 2, 8, 2),     # 2^25.6 elements at R = 32: wide
    ((4352, 10240, 16), 3, 1, 1, 7, 2),     # 272 narrow blocks for 256 CUs: wide
    ((4352, 10240, 0), 3, 1, 1, 7, 1),      # the same without LoRA: no partial sums
    ((8192, 3072, 16), 0, 0, 1, 1, 1),      # 512 narrow blocks, two even rounds: narrow
    ((8192, 3072, 32), 4, 1, 2, 4, 2),      # more than 4096 rows at R = 32: wide
    ((256, 3072, 64), 2, 1, 8, 24, 2),      # two row blocks: one span per slice
    ((1, 16, 0), 3, 1, 1, 1, 1),            # R = 0 always runs the wide kernel
])
def test_plan_choices(shape, variant, wide, rank_tiles, k_slices, launches):
    p = w4.quantize_plan(*shape)
    assert (p["variant"], p["wide"], p["rank_tiles"], p["k_slices"], p["launches"]) == \
        (variant, wide, rank_tiles, k_slices, launches), p


def test_plan_consistency_over_shapes():
    """Every plan covers K exactly once with no empty slice, fits one round on
    256 compute units when split, keeps its partial sums within the fixed
    no-alloc scratch, and needs scratch exactly when a split has LoRA."""
    for M, K, R in itertools.product([1, 17, 255, 1000, 2048, 4096, 4352, 8192, 33000],
                                     [16, 528, 3072, 12288], [0, 9, 16, 32, 64, 128]):
        p = w4.quantize_plan(M, K, R)
        nsp = -(-K // 128)
        ks, sps = p["k_slices"], p["spans_per_slice"]
        assert p["row_blocks"] == -(-M // p["rows"]) and p["grid"] == p["row_blocks"] * ks
        assert ks * sps >= nsp and (ks - 1) * sps < nsp, (M, K, R, p)
        assert R <= 16 * max(p["rank_tiles"], 1) or R == 0
        if ks > 1:
            assert p["grid"] <= 256, (M, K, R, p)
        assert 0 <= p["scratch_bytes"] <= NOALLOC
        assert (p["scratch_bytes"] > 0) == (ks > 1 and R > 0), (M, K, R, p)
        if p["scratch_bytes"]:   # 4 KiB of arrival counters, then fp32 partial sums of every slice
            assert p["scratch_bytes"] == 4096 + p["row_blocks"] * ks * p["rows"] * R * 4, (M, K, R, p)
        assert p["launches"] == (2 if p["wide"] and p["scratch_bytes"] > 0 else 1)


@pytest.mark.parametrize("shape", [(0, 3072, 16), (16, 3080, 16), (16, 3072, 129), (16, 8, 0), (1 << 20, 1 << 11, 0)])
def test_plan_rejects_invalid_sizes(shape):
    with pytest.raises(ValueError):
        w4.quantize_plan(*shape)
