"""The LDS budget solver (CPU only).

The SVDQuant W4A4 on Blackwell page (section 7) traces a +198 % throughput
loss to one buffer counted twice in a trace-time shared-memory budget: the
solver made room for memory that did not exist by cutting the main loop's
K-blocks in flight from 4 to 2, with no other symptom. Here every compiled
instance's ring depth and side region come from one constexpr solve
(w4a4_layout.hpp) that both the kernels (to carve LDS) and the host plan use.
These tests re-solve each instance's budget in a separate host program built
from the same header, once with the true counts and once with the LoRA-up
piece counted twice, and show that the miscount cannot pass unnoticed: it
changes the plan (a shallower ring, or the piece moved out of the side
region) and the kernel layouts no longer compile.
"""
import os
import subprocess

import pytest

import bit_quantized_gemm_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_gemm_amd", "csrc")


def _probe(tmp_path, factor):
    exe = tmp_path / f"budget_probe_{factor}"
    subprocess.run(["g++", "-std=c++20", "-O1", f"-DW4A4_LU_ACCOUNTING_FACTOR={factor}", f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "budget_probe.cpp"), "-o", str(exe)], check=True)

    def solve(v):
        out = subprocess.run([str(exe)] + [str(v[k]) for k in ("block_m", "block_n", "threads",
                                                               "lds_stage_bytes", "occupancy", "policy")],
                             capture_output=True, text=True, check=True).stdout.split()
        return dict(zip(("stages", "lora_place", "lds_ring_bytes", "lds_side_bytes", "lds_bytes"),
                        map(int, out)))
    return solve


def _instances():
    return [(fmt, v) for fmt in ("nvfp4", "mxfp4") for v in w4.variants(fmt)]


def test_true_counts_reproduce_every_compiled_instance(tmp_path):
    solve = _probe(tmp_path, 1)
    for fmt, v in _instances():
        got = solve(v)
        assert got == {k: v[k] for k in got}, (fmt, v["variant"], got)
        assert v["lds_bytes"] == v["lds_ring_bytes"] + v["lds_side_bytes"] <= v["lds_limit"] // v["occupancy"]
        assert v["stages"] >= 3


def test_lora_up_counted_twice_changes_the_plan(tmp_path):
    """The page's miscount: with the LoRA-up piece counted twice, the MXFP4
    256x192 instance (side region first) loses a stage in flight — 4 -> 3, the
    same symptom the page measured — and the NVFP4 128x128 side-first
    instance moves lora_up out of its side region."""
    wrong = _probe(tmp_path, 2)
    changed = {}
    for fmt, v in _instances():
        got = wrong(v)
        if got["stages"] != v["stages"] or got["lora_place"] != v["lora_place"]:
            changed[(fmt, v["block_m"], v["block_n"], v["policy"])] = (v["stages"], got["stages"],
                                                                       v["lora_place"], got["lora_place"])
    assert changed[("mxfp4", 256, 192, 1)][:2] == (4, 3)
    assert changed[("nvfp4", 128, 128, 1)][2:] == (2, 1)
    # a depth-first instance keeps its ring: a side piece never takes a stage from it
    for (fmt, bm, bn, policy), (s0, s1, _, _) in changed.items():
        if policy == 0:
            assert s1 == s0


@pytest.mark.parametrize("factor,ok", [(1, True), (2, False)])
def test_miscounted_layout_does_not_compile(tmp_path, factor, ok):
    """The kernels carve LDS from the solved budget and assert that the carved
    layout equals it; each side piece's DMA footprint is asserted against its
    count. A double-counted LoRA-up piece that is still placed therefore stops
    the build instead of silently reserving phantom LDS."""
    src = tmp_path / "instances.cpp"
    src.write_text('#include "w4a4_layout.hpp"\n'
                   "using namespace w4a4;\n"
                   "int lds[] = {Cfg256x192::LDS_BYTES, Cfg128x128::LDS_BYTES, Cfg256x128::LDS_BYTES,\n"
                   "             Cfg128x128S::LDS_BYTES, MxCfg256x192::LDS_BYTES, MxCfg128x128::LDS_BYTES};\n")
    res = subprocess.run(["g++", "-std=c++20", "-fsyntax-only", f"-DW4A4_LU_ACCOUNTING_FACTOR={factor}",
                          f"-I{CSRC}", str(src)], capture_output=True, text=True)
    assert (res.returncode == 0) == ok, res.stderr[-2000:]
    if not ok:
        assert "the carved layout is the solved budget" in res.stderr


def test_plan_reports_depth_placement_and_registers():
    """The plan at the R = 128 MLP-down shape names the ring depth, where the
    first LoRA chunk waits, and the registers of the kernel that would run."""
    p = w4.plan(4096, 3072, 12288, 128)
    assert p["stages"] == 4 and p["lora_place"] == 1
    assert p["lds_ring_bytes"] == 4 * p["lds_stage_bytes"]
    assert p["flavour"] == 1
    assert 0 < p["agprs"] <= p["vgprs"] <= p["regs_limit"] == 512
    assert p["sgprs"] > 0
    for fmt in ("nvfp4", "mxfp4"):
        for v in range(len(w4.variants(fmt))):
            q = w4.plan_variant(1000, 3072, 3072, 16, v, fmt=fmt)
            assert q["variant"] == v and 0 < q["vgprs"] <= q["regs_limit"]
