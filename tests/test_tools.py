"""Host-side measurement tooling (CPU only): the rocprofv3 summariser that
writes profiles/, bench.py's reading of the committed traffic summary, and
bench.py's refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import profsum  # noqa: E402

KNAME = "void w4a4::gemm_w4a4_kernel<w4a4::TileCfg<256, 192, 2, 2, 4, 1>, false, false>(w4a4::Params)"


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _trace_dir(tmp_path, durations, gap=0):
    """A kernel-trace run: dispatch i of the GEMM lasts durations[i] ns."""
    d = tmp_path / "trace"
    d.mkdir()
    rows, t = [], 1000
    for i, dur in enumerate(durations):
        rows.append({"Kernel_Name": KNAME, "Start_Timestamp": t, "End_Timestamp": t + dur,
                     "Grid_Size_X": 65536, "Workgroup_Size_X": 256, "LDS_Block_Size": 161792,
                     "VGPR_Count": 248, "Accum_VGPR_Count": 0, "SGPR_Count": 112, "Scratch_Size": 0})
        t += dur + gap
    # another kernel in between must not be picked up
    rows.append({**rows[0], "Kernel_Name": "void w4a4::mfma_peak_kernel<0>(int, unsigned long*)",
                 "Start_Timestamp": t, "End_Timestamp": t + 5})
    _write_csv(d / "w4_kernel_trace.csv", rows)
    _write_csv(d / "w4_kernel_stats.csv", [{"Name": KNAME, "Calls": len(durations),
                                            "AverageNs": sum(durations) / len(durations),
                                            "MinNs": min(durations), "MaxNs": max(durations),
                                            "StdDev": 0.0}])
    return d


def test_trace_timed_region_picks_the_timed_dispatches(tmp_path):
    # bench order: 1 checked call, W warm-up steps, K timed steps, 1 parity call
    W, K = 5, 4
    durations = [900] * (1 + W) + [100, 110, 120, 130] + [700]
    d = _trace_dir(tmp_path, durations)
    bench = tmp_path / "bench.json"
    bench.write_text("some log line\n" + json.dumps(
        {"warmup": W, "steps": K, "roofline": {"avg_launch_us": 0.115, "achieved": 1.0}}) + "\n")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "profsum.py"), "trace", str(d),
                          "--workload", "qkv", "--command", "cmd", "--bench-json", str(bench)],
                         cwd=ROOT, capture_output=True, text=True, check=True).stdout
    assert "dispatches 6 .. 9" in out
    row = [line for line in out.splitlines() if line.startswith("| 115.0 |")]
    assert row, out   # average of 100..130
    assert "| 115.0 | 115 | 100 | 130 | 115.0 |" in out
    assert "Median gap between consecutive launches under the tracer: 0 ns." in out


def test_trace_timed_region_counts_the_settled_warmup(tmp_path):
    # bench.py's JSON: `warmup` is the requested count, `warmup_steps_run` what
    # its settle loop ran; the timed dispatches follow the latter
    durations = [900] * (1 + 5) + [100, 110, 120, 130] + [700]
    d = _trace_dir(tmp_path, durations)
    bench = tmp_path / "bench.json"
    bench.write_text(json.dumps({"warmup": 2, "warmup_steps_run": 5, "steps": 4,
                                 "roofline": {"avg_launch_us": 0.115, "achieved": 9.0, "unit": "GB/s"}}))
    out = subprocess.run([sys.executable, os.path.join(ROOT, "profsum.py"), "trace", str(d),
                          "--workload", "qkv", "--command", "cmd", "--bench-json", str(bench)],
                         cwd=ROOT, capture_output=True, text=True, check=True).stdout
    assert "dispatches 6 .. 9" in out and "after 5 warm-up steps" in out
    assert "| 115.0 | 115 | 100 | 130 | 115.0 |" in out and "9.0 GB/s" in out


def test_trace_refuses_a_run_on_other_kernel_sources(tmp_path):
    d = _trace_dir(tmp_path, [100] * 10)
    bench = tmp_path / "bench.json"
    bench.write_text(json.dumps({"warmup": 2, "steps": 4, "roofline": {
        "avg_launch_us": 0.1, "achieved": 1.0, "kernel_source_sha256": "0123456789abcdef"}}))
    res = subprocess.run([sys.executable, os.path.join(ROOT, "profsum.py"), "trace", str(d),
                          "--workload", "qkv", "--command", "cmd", "--bench-json", str(bench)],
                         cwd=ROOT, capture_output=True, text=True)
    assert res.returncode != 0 and "profile again" in res.stderr


def test_trace_timed_region_rejects_a_short_trace(tmp_path):
    d = _trace_dir(tmp_path, [100] * 5)
    bench = tmp_path / "bench.json"
    bench.write_text(json.dumps({"warmup": 3, "steps": 4, "roofline": {"avg_launch_us": 0.1,
                                                                      "achieved": 1.0}}))
    res = subprocess.run([sys.executable, os.path.join(ROOT, "profsum.py"), "trace", str(d),
                          "--workload", "qkv", "--command", "cmd", "--bench-json", str(bench)],
                         cwd=ROOT, capture_output=True, text=True)
    assert res.returncode != 0 and "expected 4 timed dispatches" in res.stderr


def _pmc_dir(tmp_path, name, counter, copy_kib, gemm_kib):
    d = tmp_path / name
    d.mkdir()
    rows = [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
             "Counter_Value": copy_kib}]
    for i, v in enumerate(gemm_kib):
        # a counter is reported per block; the summariser sums them per dispatch
        rows.append({"Dispatch_Id": 2 + i, "Kernel_Name": KNAME, "Counter_Name": counter,
                     "Counter_Value": v / 2})
        rows.append({"Dispatch_Id": 2 + i, "Kernel_Name": KNAME, "Counter_Name": counter,
                     "Counter_Value": v / 2})
    _write_csv(d / "pmc_counter_collection.csv", rows)
    return d


def test_traffic_scales_each_counter_by_the_copy_probe(tmp_path):
    # the probe copies 256 MiB; FETCH_SIZE reads half of it (scale 2), WRITE_SIZE all of it
    f = _pmc_dir(tmp_path, "F", "FETCH_SIZE", 131072.0, [1000.0, 1100.0, 1200.0])
    w = _pmc_dir(tmp_path, "W", "WRITE_SIZE", 262144.0, [500.0, 500.0, 500.0])
    out = subprocess.run([sys.executable, os.path.join(ROOT, "profsum.py"), "traffic", str(f),
                          str(w), "--copy-mib", "256", "--workload", "qkv", "--command-fetch", "a",
                          "--command-write", "b"], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout
    vals = dict(line.split(": ") for line in out.splitlines() if not line.startswith("#"))
    assert float(vals["fetch_bytes_per_launch"]) == 2.0 * 1100.0 * 1024
    assert float(vals["write_bytes_per_launch"]) == 500.0 * 1024
    assert float(vals["hbm_bytes_per_launch"]) == (2200.0 + 500.0) * 1024
    assert vals["kernel_source_sha256"] == profsum.kernel_source_hash("nvfp4")


def test_bench_reads_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "gemm_w4a4_qkv_traffic.txt"
    assert bench.committed_traffic("qkv") is None
    path.write_text(f"# header\nkernel_source_sha256: {profsum.kernel_source_hash('nvfp4')}\n"
                    "hbm_bytes_per_launch: 12345\n")
    assert bench.committed_traffic("qkv") == 12345.0
    path.write_text("kernel_source_sha256: 0000000000000000\nhbm_bytes_per_launch: 12345\n")
    assert bench.committed_traffic("qkv") is None


def test_committed_profiles_match_the_current_kernel_sources():
    """Every summary under profiles/ names the sources it was taken on; a
    kernel change without a new profile shows up here."""
    pdir = os.path.join(ROOT, "profiles")
    for fmt, (_, prefix, _) in profsum.KERNELS.items():
        h = profsum.kernel_source_hash(fmt)
        for f in sorted(os.listdir(pdir)):
            if f.startswith(prefix + "_"):
                text = open(os.path.join(pdir, f)).read()
                assert h in text, f"{f} was taken on other {fmt} kernel sources than the current ones"


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(gpus):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_counters_labels_rocprof_derived_metrics(tmp_path):
    d = tmp_path / "D"
    d.mkdir()
    rows = []
    for i, (mu, vb) in enumerate([(47.0, 40.0), (48.0, 42.0), (49.0, 44.0)]):
        rows += [{"Dispatch_Id": 2 + i, "Kernel_Name": KNAME, "Counter_Name": "MfmaUtil", "Counter_Value": mu},
                 {"Dispatch_Id": 2 + i, "Kernel_Name": KNAME, "Counter_Name": "VALUBusy", "Counter_Value": vb}]
    _write_csv(d / "pmc_counter_collection.csv", rows)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "profsum.py"), "counters", str(d),
                          "--workload", "qkv", "--command", "cmd"], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout
    assert "derived metrics" in out and "Median over 3 dispatches" in out
    assert "| MfmaUtil | 48.000 | 100 * SQ_VALU_MFMA_BUSY_CYCLES" in out
    assert "| VALUBusy | 42.000 |" in out
