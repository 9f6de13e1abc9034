"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m bit_quantized_gemm_amd.build

writes bit_quantized_gemm_amd/libgemm_w4a4.so (the operator: include/gemm_w4a4.h)
and bit_quantized_gemm_amd/libw4a4_probes.so (measurement aids:
include/w4a4_probes.h). The kernels are compiled for gfx950 only, with
packed-fp32 VALU instructions disabled.

Each source is compiled to an object first (in parallel). For the operator
library the build then reads every kernel's resource figures (VGPRs, AGPRs,
SGPRs, LDS, spills) from the code objects inside those objects and links them
in as a table, keyed by the kernel's symbol name: the launch plan reports the
registers of the kernel it would run from the compiled code itself.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgemm_w4a4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
PROBES_LIB_PATH = os.path.join(PKG_DIR, "libw4a4_probes.so")
# library -> (the sources it is built from, whether it carries the resource table)
LIBS = {
    LIB_PATH: (("gemm_w4a4.hip", "gemm_mxfp4.hip", "w4a4_producer.hip"), True),
    PROBES_LIB_PATH: (("mfma_peak.hip", "route_probe.hip"), False),
}
ARCH = "gfx950"
LLVM = "/opt/rocm/llvm/bin"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        # keep the compiler from emitting packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag
    errs = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)


def _object(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    _run([hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
    return obj


def kernel_resources(obj: str) -> dict:
    """{kernel symbol: {vgpr, agpr, sgpr, lds, spill, scratch}} from the gfx950
    code objects in an object file's offload bundles."""
    tmp = obj + ".meta"
    os.makedirs(tmp, exist_ok=True)
    fat = os.path.join(tmp, "fatbin.bin")
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", obj], check=True)
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    blob = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(magic), blob)]
    notes = ""
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(blob)])):
        part = os.path.join(tmp, f"bundle{n}.bin")
        co = os.path.join(tmp, f"co{n}.o")
        with open(part, "wb") as f:
            f.write(blob[a:b])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={part}",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"], check=True)
        notes += subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], capture_output=True,
                                text=True, check=True).stdout
    shutil.rmtree(tmp, ignore_errors=True)
    return parse_kernel_notes(notes)


def parse_kernel_notes(notes: str) -> dict:
    """Per-kernel fields of the AMDGPU metadata note (llvm-readelf --notes)."""
    kernels, cur = {}, {}

    def flush():
        if cur.get(".name"):
            kernels[cur[".name"]] = {
                "vgpr": int(cur.get(".vgpr_count", 0)), "agpr": int(cur.get(".agpr_count", 0)),
                "sgpr": int(cur.get(".sgpr_count", 0)), "lds": int(cur.get(".group_segment_fixed_size", 0)),
                "spill": int(cur.get(".vgpr_spill_count", 0)) + int(cur.get(".sgpr_spill_count", 0)),
                "scratch": int(cur.get(".private_segment_fixed_size", 0))}

    for line in notes.splitlines():
        line = line.strip().lstrip("- ").strip()
        if ":" not in line:
            continue
        k, _, v = line.partition(":")
        k, v = k.strip(), v.strip()
        if k in (".agpr_count", ".args") and cur.get(".name"):
            flush()
            cur = {}
        cur[k] = v
    flush()
    return kernels


def _resource_source(res: dict) -> str:
    rows = "\n".join(f'    {{"{name}", {r["vgpr"]}, {r["agpr"]}, {r["sgpr"]}, {r["lds"]}, {r["spill"]}, '
                     f'{r["scratch"]}}},' for name, r in sorted(res.items()))
    return ("// Generated by bit_quantized_gemm_amd/build.py from the compiled code objects.\n"
            "#include \"w4a4_resources.h\"\n"
            "namespace w4a4 {\n"
            f"const KernelResources kKernelResources[] = {{\n{rows}\n}};\n"
            f"const int kNumKernelResources = {len(res)};\n"
            "}  // namespace w4a4\n")


def _build_one(path: str, sources, with_resources: bool, verbose: bool) -> None:
    with ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _object(s, verbose), sources))
    link = list(objs)
    if with_resources:
        res = {}
        for o in objs:
            res.update(kernel_resources(o))
        gen = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(path))[0] + "_resources.cpp")
        with open(gen, "w") as f:
            f.write(_resource_source(res))
        gobj = gen[:-4] + ".o"
        _run(["g++", "-O2", "-fPIC", "-c", f"-I{CSRC}", gen, "-o", gobj], verbose)
        link.append(gobj)
    tmp = path + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + link + ["-ldl"], verbose)
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared libraries; returns the
    operator library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    for path, (sources, with_res) in LIBS.items():
        _build_one(path, sources, with_res, verbose)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    print("\n".join(LIBS))
