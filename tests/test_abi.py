"""The C-ABI library: loads, exports what include/*.h declares, validates its
arguments, and its budget solver agrees with the compiled code objects.

CPU only: no call here reaches a kernel launch. Invalid-argument calls return
before any HIP call; the metadata check reads the library's own code object.
"""
import ctypes
import glob
import os
import re
import shutil
import subprocess

import pytest

import bit_quantized_gemm_amd as w4
from bit_quantized_gemm_amd import probes
from bit_quantized_gemm_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"


# each header and the library that must export what it declares
HEADERS = {"gemm_w4a4.h": w4.library_path, "w4a4_probes.h": probes.library_path}


def _declared_functions(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted({m.group(1) for m in re.finditer(
        r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)})


def test_every_header_is_checked():
    assert sorted(HEADERS) == sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_library_exports_every_declared_symbol(header):
    names = _declared_functions(header)
    path = HEADERS[header]()
    lib = ctypes.CDLL(path)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", path],
                        capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    assert set(names) <= exported
    if header == "gemm_w4a4.h":
        assert {"gemm_w4a4", "gemm_w4a4_f16", "gemm_mxfp4", "gemm_mxfp4_f16"} <= set(names)
        # the operator's library carries no measurement aid
        assert not any(n.startswith("w4a4_probe") for n in exported)
    else:
        assert set(names) == {"w4a4_probe_mfma_peak", "w4a4_probe_route_core", "w4a4_probe_route_b_tile"}


ENTRIES = {"bf16": w4.gemm_w4a4_raw, "f16": w4.gemm_w4a4_f16_raw,
           "mx_bf16": w4.gemm_mxfp4_raw, "mx_f16": w4.gemm_mxfp4_f16_raw}


def _call(entry="bf16", **over):
    # plausible fake device addresses: validation must reject before using them
    a = dict(act=0x10000, ascales=0x20000, wgt=0x30000, wscales=0x40000, wcscale=0x50000,
             bias=0x60000, lora_act_in=0x70000, lora_up=0x80000, out=0x90000000,
             M=64, N=64, K=128, R=16, stream=0)
    a.update(over)
    return ENTRIES[entry](a["act"], a["ascales"], a["wgt"], a["wscales"], a["wcscale"],
                            a["bias"], a["lora_act_in"], a["lora_up"], a["out"], a["M"], a["N"],
                            a["K"], a["R"], a["stream"])


@pytest.mark.parametrize("over", [
    dict(M=0), dict(N=0), dict(K=0), dict(K=8), dict(K=24), dict(R=-1), dict(M=-5),
    dict(R=w4.MAX_R + 1), dict(act=0), dict(ascales=0), dict(wgt=0), dict(wscales=0),
    dict(wcscale=0), dict(bias=0), dict(out=0), dict(lora_act_in=0), dict(lora_up=0),
    dict(M=70000, K=70000),                         # act over 2^31 bytes
    dict(M=1 << 20, N=1 << 12),                     # out over 2^31 bytes
])
@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_invalid_arguments(over, entry):
    assert _call(entry, **over) == w4.EINVAL


@pytest.mark.parametrize("over", [
    dict(act=0x10008), dict(wgt=0x30004), dict(wcscale=0x50002), dict(bias=0x60001),
    dict(out=0x90000001), dict(lora_act_in=0x70001), dict(lora_up=0x80003),
])
@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_misaligned(over, entry):
    assert _call(entry, **over) == w4.EALIGN


@pytest.mark.parametrize("K", [48, 80, 16])
@pytest.mark.parametrize("entry", ["mx_bf16", "mx_f16"])
def test_mxfp4_needs_whole_scale_blocks(K, entry):
    # the MXFP4 block is 32 values of k: a K that is a multiple of 16 only is refused
    assert _call(entry, K=K) == w4.EINVAL


@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_null_lora_allowed_without_rank_all_entries(entry):
    rc = _call(entry, R=0, lora_act_in=0, lora_up=0)
    assert rc in (w4.EDEVICE, w4.ELAUNCH, w4.OK)


def test_null_lora_allowed_without_rank():
    # with R == 0 the LoRA pointers are not needed; validation passes and only the
    # device check (no GPU here) can fail
    rc = _call(R=0, lora_act_in=0, lora_up=0)
    assert rc in (w4.EDEVICE, w4.ELAUNCH, w4.OK)
    assert rc != w4.EINVAL


@pytest.mark.parametrize("target", ["act", "ascales", "wgt", "wscales", "wcscale", "bias",
                                    "lora_act_in", "lora_up"])
@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_output_overlapping_an_input(target, entry):
    assert _call(entry, **{target: 0x90000000 + 256}) == w4.EOVERLAP


def test_strerror():
    for code in (w4.OK, w4.EINVAL, w4.EALIGN, w4.ELAUNCH, w4.EOVERLAP, w4.EDEVICE, w4.ENOMEM, w4.ESCRATCH, -99):
        assert isinstance(w4.strerror(code), str) and w4.strerror(code)


@pytest.mark.parametrize("shape", [(256, 256, 512, 32), (4096, 3072, 3072, 32),
                                   (4096, 12288, 3072, 32), (4096, 3072, 12288, 128),
                                   (1000, 3072, 3072, 16), (1, 1, 16, 0), (7, 33, 144, 3)])
def test_plan(shape):
    M, N, K, R = shape
    p = w4.plan(M, N, K, R)
    assert p["tiles_m"] * p["block_m"] >= M and (p["tiles_m"] - 1) * p["block_m"] < M
    assert p["tiles_n"] * p["block_n"] >= N and (p["tiles_n"] - 1) * p["block_n"] < N
    assert p["grid"] == p["tiles_m"] * p["tiles_n"]
    assert p["k_stages"] == -(-K // p["block_k"])
    assert p["lora_steps"] == -(-R // 16)
    assert p["lds_bytes"] <= p["lds_limit"] == 163840
    assert p["threads"] == 64 * p["waves_m"] * p["waves_n"] * p["k_groups"]
    with pytest.raises(ValueError):
        w4.plan(M, N, K + 8, R)


@pytest.mark.parametrize("shape", [(256, 256, 512, 32), (4096, 3072, 3072, 32),
                                   (4096, 12288, 3072, 32), (4352, 3840, 15360, 128),
                                   (1000, 3072, 3072, 16), (1, 1, 32, 0), (7, 33, 160, 3)])
def test_plan_mxfp4(shape):
    M, N, K, R = shape
    p = w4.plan(M, N, K, R, fmt="mxfp4")
    assert p["block_k"] == 128
    assert p["tiles_m"] * p["block_m"] >= M and (p["tiles_m"] - 1) * p["block_m"] < M
    assert p["tiles_n"] * p["block_n"] >= N and (p["tiles_n"] - 1) * p["block_n"] < N
    assert p["grid"] == p["tiles_m"] * p["tiles_n"]
    assert p["k_stages"] == -(-K // 128)
    assert p["lds_bytes"] <= p["lds_limit"] == 163840
    with pytest.raises(ValueError):
        w4.plan(M, N, K + 16, R, fmt="mxfp4")
    with pytest.raises(ValueError):
        w4.plan(M, N, K, R, fmt="int4")


def test_plan_prefers_full_chip_at_qkv():
    # 4096 x 3072 in 256 x 192 tiles is exactly one tile per compute unit
    p = w4.plan(4096, 3072, 3072, 32)
    assert (p["block_m"], p["block_n"]) == (256, 192) and p["grid"] == 256


def _code_object_metadata():
    lib = w4.library_path()
    tmp = os.path.join(ROOT, "_build_meta")
    os.makedirs(tmp, exist_ok=True)
    fat = os.path.join(tmp, "fatbin.bin")
    co = os.path.join(tmp, "co.o")
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", lib],
                   check=True)
    # one offload bundle per translation unit, concatenated in the section
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    blob = open(fat, "rb").read()
    starts = [i for i in range(len(blob)) if blob.startswith(magic, i)]
    assert starts, "no offload bundle in the library"
    notes = ""
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(blob)])):
        part = os.path.join(tmp, f"bundle{n}.bin")
        with open(part, "wb") as f:
            f.write(blob[a:b])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                        f"--input={part}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--output={co}"], check=True)
        notes += subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], capture_output=True,
                                text=True, check=True).stdout
    shutil.rmtree(tmp, ignore_errors=True)
    kernels = {}
    cur = {}
    for line in notes.splitlines():
        line = line.strip().lstrip("- ").strip()
        if ":" not in line:
            continue
        k, _, v = line.partition(":")
        k, v = k.strip(), v.strip()
        if k in (".agpr_count", ".args") and cur.get(".name"):
            kernels[cur[".name"]] = cur
            cur = {}
        cur[k] = v
    if cur.get(".name"):
        kernels[cur[".name"]] = cur
    return kernels


@pytest.mark.skipif(not os.path.exists(f"{LLVM}/clang-offload-bundler"), reason="no ROCm llvm")
def test_solver_lds_matches_code_objects():
    """The LDS bytes the solver budgets equal what the compiler reserved
    (ratio 1.000) for every compiled instance; the register count allows the
    occupancy each instance is budgeted for; nothing spills inside a kernel
    that the solver may pick for a full-chip workload."""
    meta = _code_object_metadata()
    assert meta, "no kernels found in the code object"
    # mangled tile configurations: w4a4::TileCfg (NVFP4) and w4a4::MxTileCfg (MXFP4)
    # instances per tile: NVFP4 {general, fast, fast with byte-wise act
    # scales} x {bf16, fp16}; MXFP4 {general, fast} x {bf16, fp16}, plus fast
    # with act-scale windows where the 256-row tile's scale rounds have room;
    # the 64x192 k-group tile (NVFP4) and the 128x128 tile (MXFP4) also in K
    # slices (fast, bf16 and fp16)
    cases = [(v, "7TileCfgI", 8 if (v["block_m"], v["k_groups"]) == (64, 2) else 6) for v in w4.variants("nvfp4")] + \
            [(v, "9MxTileCfgI", 6 if v["block_m"] == 256 else 6) for v in w4.variants("mxfp4")]
    for v, tag, count in cases:
        key = tag + "Li%dELi%dELi%dELi%dELi%dELi%dE" % (v["block_m"], v["block_n"], v["waves_m"],
                                                       v["waves_n"], v["occupancy"], v["policy"])
        hits = [m for n, m in meta.items() if key in n]
        assert len(hits) == count, (key, list(meta))
        for m in hits:
            assert int(m[".group_segment_fixed_size"]) == v["lds_bytes"], (key, m)
            assert int(m[".vgpr_spill_count"]) == 0, (key, m)
            assert int(m.get(".private_segment_fixed_size", 0)) == 0, (key, m)
            regs = int(m[".vgpr_count"])
            waves_per_simd = max(1, (v["waves_m"] * v["waves_n"] * v["k_groups"] + 3) // 4)
            occ = v["lds_limit"] // v["lds_bytes"]
            assert regs * waves_per_simd <= 512, (key, regs)
            assert occ >= 1


@pytest.mark.parametrize("kind,iters,clocks,want", [
    (3, 16, 0x1000, w4.EINVAL), (-1, 16, 0x1000, w4.EINVAL), (0, 0, 0x1000, w4.EINVAL),
    (1, 16, 0, w4.EINVAL), (2, 16, 0x1004, w4.EALIGN)])
def test_mfma_peak_validation(kind, iters, clocks, want):
    assert probes.mfma_peak_raw(kind, iters, clocks, 0) == want


@pytest.mark.parametrize("route,blocks,clocks,want", [
    (2, 16, 0x1000, w4.EINVAL), (-1, 16, 0x1000, w4.EINVAL), (0, 0, 0x1000, w4.EINVAL),
    (1, 16, 0, w4.EINVAL), (0, 16, 0x1004, w4.EALIGN)])
def test_route_core_validation(route, blocks, clocks, want):
    assert probes.route_core_raw(route, blocks, clocks, 0) == want


_TILE = (0x1000, 0x2000, 0x3000, 0x4000, 0x5000)   # act, ascales, wgt, wscales, out


@pytest.mark.parametrize("ptrs,K,want", [
    (_TILE, 8, w4.EINVAL), (_TILE, 24, w4.EINVAL), (_TILE, 0, w4.EINVAL),
    (_TILE, 65536 + 16, w4.EINVAL),
    ((0,) + _TILE[1:], 64, w4.EINVAL), (_TILE[:4] + (0,), 64, w4.EINVAL),
    (_TILE[:1] + (0,) + _TILE[2:], 64, w4.EINVAL),
    ((0x1002,) + _TILE[1:], 64, w4.EALIGN), (_TILE[:2] + (0x3001,) + _TILE[3:], 64, w4.EALIGN),
    (_TILE[:4] + (0x5002,), 64, w4.EALIGN)])
def test_route_b_tile_validation(ptrs, K, want):
    assert probes.route_b_tile_raw(*ptrs, K, 0) == want


@pytest.mark.parametrize("fmt,out_f16,variant", [("nvfp4", 0, 99), ("nvfp4", 0, -2), ("mxfp4", 1, 7),
                                                 ("nvfp4", 2, 0)])
def test_run_rejects_unknown_variant_or_type(fmt, out_f16, variant):
    rc = w4.run_raw(fmt, out_f16, variant, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000,
                    0x70000, 0x80000, 0x90000000, 64, 64, 128, 16, 0)
    assert rc == w4.EINVAL


def test_run_rejects_unknown_format():
    lib = _native.load()
    assert lib.gemm_w4a4_run(5, 0, -1, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000,
                             0x70000, 0x80000, 0x90000000, 64, 64, 128, 16, None) == w4.EINVAL


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_plan_variant_matches_plan(fmt):
    for shape in [(4096, 3072, 3072, 32), (1000, 3072, 3072, 16), (4352, 3840, 3840, 128)]:
        assert w4.plan_variant(*shape, -1, fmt=fmt) == w4.plan(*shape, fmt=fmt)
        for v in range(len(w4.variants(fmt))):
            q = w4.plan_variant(*shape, v, fmt=fmt)
            assert q["variant"] == v and q["grid"] == q["tiles_m"] * q["tiles_n"]
    with pytest.raises(ValueError):
        w4.plan_variant(64, 64, 128, 0, len(w4.variants(fmt)), fmt=fmt)


# ---------------------------------------------------------------- quantize_w4a4_act

QENTRIES = ["quantize_raw", "quantize_noalloc_raw"]   # quantize_w4a4_act and its no-allocation twin


def _q(qentry="quantize_raw", **over):
    a = dict(x=0x10000, lora_down=0x200000, act=0x300000, ascales=0x400000, lora_act_in=0x500000,
             M=64, K=128, R=16, stream=0)
    a.update(over)
    return getattr(w4, qentry)(a["x"], a["lora_down"], a["act"], a["ascales"], a["lora_act_in"],
                               a["M"], a["K"], a["R"], a["stream"])


@pytest.mark.parametrize("over", [dict(M=0), dict(K=0), dict(K=8), dict(K=24), dict(R=-1),
                                  dict(R=w4.QUANTIZE_MAX_R + 1), dict(x=0), dict(act=0),
                                  dict(ascales=0), dict(lora_down=0), dict(lora_act_in=0),
                                  dict(M=1 << 20, K=1 << 11)])
@pytest.mark.parametrize("qentry", QENTRIES)
def test_quantize_invalid_arguments(over, qentry):
    assert _q(qentry, **over) == w4.EINVAL


@pytest.mark.parametrize("over", [dict(x=0x10008), dict(lora_down=0x200004), dict(act=0x300004),
                                  dict(lora_act_in=0x500001)])
@pytest.mark.parametrize("qentry", QENTRIES)
def test_quantize_misaligned(over, qentry):
    assert _q(qentry, **over) == w4.EALIGN


@pytest.mark.parametrize("over", [dict(act=0x10000 + 64), dict(ascales=0x200000 + 16),
                                  dict(lora_act_in=0x300000 + 32), dict(ascales=0x300000 + 8)])
@pytest.mark.parametrize("qentry", QENTRIES)
def test_quantize_overlap(over, qentry):
    assert _q(qentry, **over) == w4.EOVERLAP


@pytest.mark.parametrize("qentry", QENTRIES)
def test_quantize_rank_zero_needs_no_lora_pointers(qentry):
    rc = _q(qentry, R=0, lora_down=0, lora_act_in=0)
    assert rc in (w4.EDEVICE, w4.ELAUNCH, w4.OK)


@pytest.mark.skipif(not os.path.exists(f"{LLVM}/clang-offload-bundler"), reason="no ROCm llvm")
def test_no_kernel_spills():
    """No compiled kernel of the operator library spills registers or uses
    scratch memory (the build's resource table, read from the code objects)."""
    from bit_quantized_gemm_amd.build import BUILD_DIR
    src = open(os.path.join(BUILD_DIR, "libgemm_w4a4_resources.cpp")).read()
    rows = re.findall(r'\{"(\w+)", (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\}', src)
    # the producer: three narrow kernels, the wide kernel and its two reductions
    assert len(rows) >= 38 and sum("producer_" in r[0] for r in rows) >= 6
    for name, vgpr, agpr, sgpr, lds, spill, scratch in rows:
        assert int(spill) == 0 and int(scratch) == 0, name
