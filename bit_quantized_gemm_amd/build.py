"""Build the gfx950 shared library in-tree with hipcc.

    python -m bit_quantized_gemm_amd.build

writes bit_quantized_gemm_amd/libgemm_w4a4.so. The kernels are compiled for
gfx950 only, with packed-fp32 VALU instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgemm_w4a4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(CSRC, f) for f in ("gemm_w4a4.hip", "gemm_mxfp4.hip", "mfma_peak.hip", "route_probe.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
        # keep the compiler from emitting packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared library; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag
    errs = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
