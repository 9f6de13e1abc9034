"""The C ABI from plain C: include/gemm_w4a4.h compiles as strict C11 with gcc
(-Wall -Wextra -Werror, no HIP or torch headers), and a program linked
against libgemm_w4a4.so gets the documented results from the calls that need
no GPU (tests/c_consumer.c)."""
import os
import shutil
import subprocess

import pytest

from bit_quantized_gemm_amd.build import LIB_PATH, PKG_DIR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_c_program_uses_the_c_abi(tmp_path):
    assert os.path.exists(LIB_PATH), "build the library first"
    exe = tmp_path / "c_consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_consumer.c"),
           "-o", str(exe), f"-L{PKG_DIR}", "-lgemm_w4a4", f"-Wl,-rpath,{PKG_DIR}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and run.stdout.count("ok") >= 14, run.stdout
    # the binding's ctypes mirrors of the plan structs have the C layout's size
    import ctypes

    from bit_quantized_gemm_amd._native import Plan, QuantizePlan
    sizes = dict(line.rsplit(" ", 1) for line in run.stdout.splitlines() if line.startswith("sizeof"))
    assert int(sizes["sizeof gemm_w4a4_plan_t"]) == ctypes.sizeof(Plan)
    assert int(sizes["sizeof quantize_w4a4_plan_t"]) == ctypes.sizeof(QuantizePlan)
