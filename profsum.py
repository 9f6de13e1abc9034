"""Summaries of rocprofv3 runs of the W4A4 kernels, as short text files.

    python profsum.py trace DIR --workload qkv --command "..."
    python profsum.py traffic FETCH_DIR WRITE_DIR --copy-mib 256 \
        --workload qkv --command "..."
    python profsum.py counters DIR --workload qkv --command "..."

`trace` reads the kernel statistics of a `--kernel-trace --stats` run; given
the JSON line bench.py printed in that run (`--bench-json`), it also gives the
statistics of the timed region's dispatches alone (rocprofv3's own averages
include the warm-up, whose first launches run before the clock has settled).
`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a program
that also made one device copy of COPY_MIB MiB (bench.py --copy-probe-mb): each
counter is scaled by (true bytes of that copy) / (what the counter read for
it), and the GEMM's HBM bytes per launch are the scaled median over its
dispatches (per kernel name, summed: a producer step with a split K is two
launches). `counters` tabulates the counters of one `--pmc` run. `--fmt mxfp4`
selects the MXFP4 kernel, `--fmt producer` the activation producer's kernels
(default: the NVFP4 GEMM).
The file carries the hash of the kernel sources it was taken on, so a reader
(bench.py) can tell whether it still describes the current kernel. That hash
is the one bench.py recorded in the profiled run's JSON line (`--bench-json`,
or `--bench-out` for a counter run's output): a run whose kernel sources
differ from the current ones is refused, not summarised under the current
hash.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_quantized_gemm_amd", "csrc")
_SHARED = ("w4a4_common.hpp", "w4a4_epilogue.hpp", "w4a4_layout.hpp")
# per format: (kernel name tag, summary file prefix, the sources the kernel is built from)
KERNELS = {
    "nvfp4": ("gemm_w4a4_kernel", "gemm_w4a4", ("gemm_w4a4.hip",) + _SHARED),
    "mxfp4": ("gemm_mxfp4_kernel", "gemm_mxfp4", ("gemm_mxfp4.hip",) + _SHARED),
    "producer": ("producer_", "quantize_w4a4_act",
                 ("w4a4_producer.hip", "w4a4_common.hpp", "w4a4_host.hpp", "w4a4_layout.hpp")),
}
COPY_TAG = "copyBuffer"


def kernel_source_hash(fmt: str = "nvfp4") -> str:
    """First 16 hex digits of the sha256 over one kernel's sources."""
    h = hashlib.sha256()
    for f in KERNELS[fmt][2]:
        p = os.path.join(_CSRC, f)
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _bench_line(path: str) -> dict:
    """The last JSON line bench.py printed into `path`."""
    b = None
    with open(path) as f:
        for line in f:
            if line.lstrip().startswith("{"):
                b = json.loads(line)
    if b is None:
        raise SystemExit(f"no JSON line in {path}")
    return b


def _check_sources(path, fmt: str) -> None:
    """Refuse a profiled run whose recorded kernel sources are not the current ones."""
    if path is None:
        return
    rec = _bench_line(path).get("roofline", {}).get("kernel_source_sha256")
    if rec is not None and rec != kernel_source_hash(fmt):
        raise SystemExit(f"{path}: the profiled run used kernel sources {rec}, the current ones are "
                         f"{kernel_source_hash(fmt)}: profile again")


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _per_dispatch(directory: str):
    """{dispatch id: (kernel name, {counter: summed value})} of a --pmc run."""
    path = _one(os.path.join(directory, "*counter_collection.csv"))
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], defaultdict(float)))
        vals[r["Counter_Name"]] += float(r["Counter_Value"])
    return dict(sorted(out.items()))


def trace(args) -> str:
    tag, name, _ = KERNELS[args.fmt]
    tag = args.tag or tag
    _check_sources(args.bench_json, args.fmt)
    stats = list(csv.DictReader(open(_one(os.path.join(args.dir, "*kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(args.dir, "*kernel_trace.csv")))))
    g = [r for r in rows if tag in r["Kernel_Name"]]
    lines = [f"# {name} kernel trace, {args.workload} workload", "",
             "Command (repository root, one MI355X, library built in-tree):", "",
             f"    {args.command}", "",
             f"Kernel source sha256[:16]: {kernel_source_hash(args.fmt)}", "",
             "| Kernel | Calls | Average ns | Min ns | Max ns | StdDev ns |",
             "|---|---|---|---|---|---|"]
    for s in stats:
        lines.append(f"| `{s['Name'][:110]}` | {s['Calls']} | {float(s['AverageNs']):.1f} | "
                     f"{s['MinNs']} | {s['MaxNs']} | {float(s['StdDev']):.1f} |")
    if g:
        r = g[0]
        lines += ["", f"Launch: grid {r['Grid_Size_X']} work-items / workgroup {r['Workgroup_Size_X']}, "
                      f"LDS {r['LDS_Block_Size']} B, VGPR {r['VGPR_Count']}, AGPR {r['Accum_VGPR_Count']}, "
                      f"SGPR {r['SGPR_Count']}, scratch {r['Scratch_Size']} B."]
        gs = sorted(g, key=lambda r: int(r["Start_Timestamp"]))
        gaps = [int(b["Start_Timestamp"]) - int(a["End_Timestamp"]) for a, b in zip(gs, gs[1:])]
        if gaps:
            lines.append(f"Median gap between consecutive launches under the tracer: "
                         f"{statistics.median(gaps):.0f} ns.")
        if args.bench_json:
            lines += timed_region(gs, args.bench_json)
    return "\n".join(lines) + "\n"


def timed_region(gs, bench_json: str) -> list:
    """Statistics of the timed region's dispatches. bench.py launches the
    kernel once through the checked binding, then its untimed warm-up steps
    (`warmup_steps_run`: the requested `warmup`, continued until the clock has
    settled), then the `steps` timed ones (then one more for its parity
    sample). A step is one dispatch of the selected kernel."""
    b = _bench_line(bench_json)
    warm = int(b.get("warmup_steps_run", b["warmup"]))
    first, k = 1 + warm, int(b["steps"])
    sel = gs[first:first + k]
    if len(sel) != k:
        raise SystemExit(f"expected {k} timed dispatches after {first}, found {len(sel)}")
    d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel]
    span = int(sel[-1]["End_Timestamp"]) - int(sel[0]["Start_Timestamp"])
    return ["", f"Timed region of that bench run: dispatches {first} .. {first + k - 1} of the kernel "
                f"({k} launches after {warm} warm-up steps):", "",
            "| Average ns | Median ns | Min ns | Max ns | Span / launches ns |", "|---|---|---|---|---|",
            f"| {statistics.mean(d):.1f} | {statistics.median(d):.0f} | {min(d)} | {max(d)} | {span / k:.1f} |",
            "", f"bench.py's own figure in that run (HIP events at the ends of the timed region): "
                f"{b['roofline']['avg_launch_us'] * 1e3:.0f} ns per step, "
                f"{b['roofline']['achieved']:.1f} {b['roofline'].get('unit', 'TFLOP/s')}."]


def traffic(args) -> str:
    tag, name, _ = KERNELS[args.fmt]
    for out in args.bench_out or []:
        _check_sources(out, args.fmt)
    fetch, write = _per_dispatch(args.fetch_dir), _per_dispatch(args.write_dir)
    true_kib = args.copy_mib * 1024.0

    def scale(runs, counter):
        copies = [v[counter] for n, v in runs.values() if COPY_TAG in n]
        if not copies:
            raise SystemExit(f"no copy dispatch found for {counter}")
        probe = max(copies)   # the probe is by far the largest copy
        per_kernel = defaultdict(list)
        for n, v in runs.values():
            if tag in n:
                per_kernel[n].append(v[counter])
        if not per_kernel:
            raise SystemExit(f"no {tag} dispatch found for {counter}")
        med = sum(statistics.median(x) for x in per_kernel.values())   # one launch of each per step
        return probe, true_kib / probe, med, min(len(x) for x in per_kernel.values())

    fp, ff, fg, fn = scale(fetch, "FETCH_SIZE")
    wp, wf, wg, wn = scale(write, "WRITE_SIZE")
    fetch_b, write_b = fg * ff * 1024.0, wg * wf * 1024.0
    lines = [f"# {name} HBM traffic per launch, {args.workload} workload",
             "# Commands (repository root, one MI355X, library built in-tree):",
             f"#   {args.command_fetch}", f"#   {args.command_write}",
             f"# copy probe: one device copy of {args.copy_mib} MiB = {true_kib:.0f} KiB read and written",
             f"# FETCH_SIZE read {fp:.1f} KiB for the probe -> scale {ff:.4f}; "
             f"kernel median over {fn} dispatches {fg:.1f} KiB",
             f"# WRITE_SIZE read {wp:.1f} KiB for the probe -> scale {wf:.4f}; "
             f"kernel median over {wn} dispatches {wg:.1f} KiB",
             f"kernel_source_sha256: {kernel_source_hash(args.fmt)}",
             f"fetch_bytes_per_launch: {fetch_b:.0f}",
             f"write_bytes_per_launch: {write_b:.0f}",
             f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}"]
    return "\n".join(lines) + "\n"


# rocprofv3's derived metrics used here, as its counter listing defines them
# (sums over the device, GRBM_GUI_ACTIVE the maximum over its instances).
DERIVED = {
    "MfmaUtil": "100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMD count): % of SIMD time the matrix core is busy",
    "VALUBusy": "100 * SQ_ACTIVE_INST_VALU / (CU count * GRBM_GUI_ACTIVE): % of time vector ALU instructions are processed",
    "LDSBankConflict": "100 * SQ_LDS_BANK_CONFLICT / (GRBM_GUI_ACTIVE * CU count): % of time the LDS stalls on bank conflicts",
    "LdsUtil": "100 * SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE * CU count): % of time the LDS is busy",
    "LdsBankConflict": "SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT): conflict cycles per LDS access cycle",
    "VmemLatency": "accumulated SQ_INST_LEVEL_VMEM / SQ_INSTS_VMEM: average cycles a vector memory instruction is in flight",
    "LdsLatency": "accumulated SQ_INST_LEVEL_LDS / SQ_INSTS_LDS: average cycles an LDS instruction is in flight",
    "MemUnitStalled": "100 * TCP_TCP_TA_DATA_STALL_CYCLES (max) / GRBM_GUI_ACTIVE / SE count: % of time the memory unit is stalled",
}


def counters(args) -> str:
    tag, name, _ = KERNELS[args.fmt]
    for out in args.bench_out or []:
        _check_sources(out, args.fmt)
    runs = _per_dispatch(args.dir)
    g = [v for n, v in runs.values() if tag in n]
    names = sorted(g[0]) if g else []
    derived = bool(names) and all(c in DERIVED for c in names)
    title = "rocprofv3 derived metrics" if derived else "hardware counters"
    what = ("values as rocprofv3 computes them per dispatch" if derived
            else "values summed over the device")
    lines = [f"# {name} {title}, {args.workload} workload", "",
             "Command (repository root, one MI355X, library built in-tree):", "",
             f"    {args.command}", "",
             f"Kernel source sha256[:16]: {kernel_source_hash(args.fmt)}", "",
             f"Median over {len(g)} dispatches ({what}):", ""]
    if derived:
        lines += ["| Metric | Value | Definition |", "|---|---|---|"]
        for c in names:
            lines.append(f"| {c} | {statistics.median(v[c] for v in g):.3f} | {DERIVED[c]} |")
    else:
        lines += ["| Counter | Value |", "|---|---|"]
        for c in names:
            lines.append(f"| {c} | {statistics.median(v[c] for v in g):.0f} |")
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="profsum")
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--bench-json", default=None, help="bench.py's output of the traced run")
    t.add_argument("--tag", default=None, help="kernel-name substring of the launch to time (default: the format's)")
    f = sub.add_parser("traffic")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("--copy-mib", type=float, required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--command-fetch", required=True)
    f.add_argument("--command-write", required=True)
    f.add_argument("--bench-out", nargs="*", help="bench.py's output of the profiled runs (source check)")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--bench-out", nargs="*", help="bench.py's output of the profiled run (source check)")
    for p in (t, f, c):
        p.add_argument("--fmt", default="nvfp4", choices=sorted(KERNELS))
    a = ap.parse_args(argv)
    sys.stdout.write({"trace": trace, "traffic": traffic, "counters": counters}[a.what](a))
    return 0


if __name__ == "__main__":
    sys.exit(main())
