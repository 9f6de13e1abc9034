"""The producer's explicit lora_down loads (CPU only; reads the gfx950 assembly).

quantize_w4a4_act issues its lora_down loads as explicit buffer_load_dwordx4
into registers, which the compiler does not track (tracked loads would make it wait for every
outstanding memory op, the DMA ring included, while stores are in flight). The
kernel then owns the synchronisation: between such a load and the s_waitcnt
that guarantees its completion, no instruction may read or write the load's
destination registers (the compiler, not knowing the load is still in flight,
could otherwise copy or reuse them). This test compiles the kernel source to
assembly and walks every such load forward to its wait.
"""
import os
import re
import subprocess

import pytest

from bit_quantized_gemm_amd import build as B

SRC = os.path.join(B.CSRC, "w4a4_producer.hip")
VMEM = ("global_load", "global_store", "buffer_", "flat_", "scratch_")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _split(line):
    body = line.split(";")[0].strip()
    parts = body.split(None, 1)
    if not parts:
        return "", []
    return parts[0], ([t.strip() for t in re.split(r",\s*", parts[1])] if len(parts) > 1 else [])


def _successors(code, j, labels):
    op, ops = _split(code[j])
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels.get(ops[0], len(code))]
    if op.startswith("s_cbranch"):
        return [j + 1, labels.get(ops[0], len(code))]
    return [j + 1]


def _check_kernel(code):
    """Returns (loads checked, violations) for one kernel's lines. From each
    load into registers, every control-flow path is followed until an
    s_waitcnt whose vmcnt covers the load (the number of vector-memory ops
    issued after it on that path)."""
    labels = {l.split(":")[0]: i for i, l in enumerate(code) if re.match(r"^\.LBB\S+:", l)}
    bad, n = [], 0
    for i, line in enumerate(code):
        op, ops = _split(line)
        # a load into registers (the ring's DMAs write LDS: their first operand is an offset)
        if op != "buffer_load_dwordx4" or re.search(r"\blds\b", line):
            continue
        n += 1
        dst = _regs(ops[0])
        stack, seen = [(j, 0) for j in _successors(code, i, labels)], set()
        while stack:
            j, after = stack.pop()
            if j >= len(code) or (j, after) in seen:
                continue
            seen.add((j, after))
            op2, ops2 = _split(code[j])
            if op2.startswith("s_waitcnt"):
                m = re.search(r"vmcnt\((\d+)\)", code[j])
                if m and int(m.group(1)) <= after:
                    continue
            if not op2.startswith("s_") and any(_regs(t) & dst for t in ops2):
                bad.append((line.strip(), code[j].strip()))
                break
            if op2.startswith(VMEM):
                after = min(after + 1, 64)
            stack.extend((k, after) for k in _successors(code, j, labels))
    return n, bad


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "producer.s"
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-std=c++20", "--offload-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{B.INCLUDE}", f"-I{B.CSRC}", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text().splitlines()


def test_no_register_touched_while_its_load_is_in_flight(asm):
    # the narrow kernels (R = 0, <= 16, <= 32) load lora_down untracked; the
    # wide kernel moves every operand by DMA into LDS
    starts = [i for i, l in enumerate(asm) if re.match(r"^_ZN4w4a415producer_kernel\S*:", l)]
    assert len(starts) >= 2
    total = 0
    for s in starts:
        e = next(i for i in range(s, len(asm)) if "s_endpgm" in asm[i])
        n, bad = _check_kernel(asm[s:e])
        assert not bad, (asm[s], bad[:3])
        total += n
    assert total > 0
