"""The seeded generators follow the stated input recipe (CPU only)."""
import numpy as np
import pytest

import synthetic


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_recipe(name):
    wl = synthetic.workload(name)
    x = synthetic.make_inputs(name)
    M, N, K, R = wl.shape
    assert x["act"].shape == (M, K // 2) and x["act"].dtype == np.uint8
    assert x["wgt"].shape == (N, K // 2)
    assert x["ascales"].shape == (K // 16, M) and x["wscales"].shape == (K // 16, N)
    assert x["lora_act_in"].shape == (M, R) and x["lora_up"].shape == (R, N)
    # nibbles uniform over all 16 codes, independently in both halves
    for half in (x["act"] & 15, x["act"] >> 4):
        counts = np.bincount(half.ravel(), minlength=16) / half.size
        assert np.all(np.abs(counts - 1 / 16) < 0.01)
    # scales: exponent field 3..9 (2^-4..2^2), any mantissa, optional exact zeros
    for s in (x["ascales"], x["wscales"]):
        nz = s[s != 0]
        assert np.all((nz >> 7) == 0)
        e = (nz >> 3) & 15
        assert e.min() == 3 and e.max() == 9
        assert set(np.unique(nz & 7)) == set(range(8))
        frac0 = np.mean(s == 0)
        assert abs(frac0 - wl.zero_scale_frac) < 0.01
    assert np.all((x["wcscale"] >= 0.5) & (x["wcscale"] < 1.5))
    assert abs(np.mean(x["bias"] == 0) - wl.zero_bias_frac) < 0.01 + 1e-9
    la = (x["lora_act_in"].astype(np.uint32) << 16).view(np.float32)
    assert abs(la.std() - wl.lora_act_std) < 0.2 * wl.lora_act_std


def test_seed_is_fixed():
    a = synthetic.make_inputs("tiny")
    b = synthetic.make_inputs("tiny")
    assert all(np.array_equal(a[k], b[k]) for k in ("act", "ascales", "lora_up", "bias"))


def test_bf16_bits_rne():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5], np.float32)
    assert list(synthetic.bf16_bits_from_f32(v)) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_recipe_mxfp4(name):
    wl = synthetic.workload(name)
    x = synthetic.make_inputs(name, fmt="mxfp4")
    M, N, K, R = wl.shape
    assert x["ascales"].shape == (K // 32, M) and x["wscales"].shape == (K // 32, N)
    for s in (x["ascales"], x["wscales"]):
        nz = s[s != 0]
        # UE8M0 127 + e, e uniform in -4..2; "zero" blocks use the smallest scale 0x00
        assert set(np.unique(nz)) == set(range(123, 130))
        assert abs(np.mean(s == 0) - wl.zero_scale_frac) < 0.01
    for half in (x["act"] & 15, x["act"] >> 4):
        counts = np.bincount(half.ravel(), minlength=16) / half.size
        assert np.all(np.abs(counts - 1 / 16) < 0.01)


def test_recipe_f16_lora_same_draws():
    a = synthetic.make_inputs("tiny", dtype="bf16")
    b = synthetic.make_inputs("tiny", dtype="f16")
    assert all(np.array_equal(a[k], b[k]) for k in ("act", "ascales", "wgt", "wscales", "bias"))
    la16 = b["lora_act_in"].view(np.float16).astype(np.float32)
    la_bf = (a["lora_act_in"].astype(np.uint32) << 16).view(np.float32)
    # both round the same float32 draws: within one bf16 ulp of each other
    assert np.all(np.abs(la16 - la_bf) <= np.abs(la_bf) * 2.0 ** -7 + 2.0 ** -24)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_large_inputs_recipe(fmt):
    x = synthetic.large_inputs(512, 64, 1024, 16, seed=3, fmt=fmt)
    kb = 1024 // (16 if fmt == "nvfp4" else 32)
    assert x["act"].shape == (512, 512) and x["ascales"].shape == (kb, 512)
    for half in (x["act"] & 15, x["act"] >> 4):
        counts = np.bincount(half.ravel(), minlength=16) / half.size
        assert np.all(np.abs(counts - 1 / 16) < 0.01)
    for s in (x["ascales"], x["wscales"]):
        if fmt == "nvfp4":
            assert set(np.unique((s >> 3) & 15)) == set(range(3, 10)) and np.all(s >> 7 == 0)
            assert set(np.unique(s & 7)) == set(range(8))
        else:
            assert set(np.unique(s)) == set(range(123, 130))
