"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m bit_quantized_gemm_amd.build

writes bit_quantized_gemm_amd/libgemm_w4a4.so (the operator: include/gemm_w4a4.h)
and bit_quantized_gemm_amd/libw4a4_probes.so (measurement aids:
include/w4a4_probes.h). The kernels are compiled for gfx950 only, with
packed-fp32 VALU instructions disabled.
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
PROBES_LIB_PATH = os.path.join(PKG_DIR, "libw4a4_probes.so")
# library -> the sources it is built from
LIBS = {
    LIB_PATH: ("gemm_w4a4.hip", "gemm_mxfp4.hip"),
    PROBES_LIB_PATH: ("mfma_peak.hip", "route_probe.hip"),
}
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


def _build_one(path: str, sources, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-o", tmp] + [os.path.join(CSRC, f) for f in sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag
    errs = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared libraries; returns the
    operator library's path."""
    for path, sources in LIBS.items():
        _build_one(path, sources, verbose)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    print("\n".join(LIBS))
