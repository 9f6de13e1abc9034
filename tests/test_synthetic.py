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
