"""The solver's choice of compiled tile instance against measured timings.
Needs a gfx950 GPU.

gemm_w4a4 and gemm_mxfp4 pick a compiled instance per shape from rounds of
tiles and a table of relative costs per output element (one per instance),
or split the rows between two instances launched in turn. This test times
every instance of the format over the whole shape, and the solver's own
plan, at shapes where the choice matters (few rows, one round, several
rounds, the pages' production shape, where the plan splits) and requires the
plan to be within 15 % of the fastest single instance: a kernel change that
moves an instance's real cost far from its table entry fails here. (The margin covers run-to-run spread and near-ties; `bench.py
--calibrate` prints the measured costs.)"""
import time

import numpy as np
import pytest
import torch

import bit_quantized_gemm_amd as w4
import synthetic

from gpu_helpers import DEV, _say, to_device

pytestmark = pytest.mark.gpu

CASES = [("nvfp4", "ragged"), ("nvfp4", "qkv"), ("nvfp4", "prod_k3840_n3072"), ("nvfp4", (2000, 3072, 3072, 16)),
         ("mxfp4", "ragged"), ("mxfp4", "qkv"), ("mxfp4", "prod_k3840_n3072")]


def time_instances(fmt, x, rounds=3, reps=20, warm_ms=40.0):
    """Best average time (us) of every compiled instance of `fmt` over the
    whole shape, and (key -1) of the solver's plan."""
    d = to_device(x)
    M, N, K, R = x["M"], x["N"], x["K"], x["R"]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.current_stream()
    ptr = lambda t: 0 if t is None else t.data_ptr()
    args = (ptr(d["act"]), ptr(d["ascales"]), ptr(d["wgt"]), ptr(d["wscales"]), ptr(d["wcscale"]),
            ptr(d["bias"]), ptr(d["lora_act_in"]), ptr(d["lora_up"]), out.data_ptr(), M, N, K, R,
            stream.cuda_stream)
    variants = list(range(len(w4.variants(fmt)))) + [-1]

    def run(v, n):
        for _ in range(n):
            rc = w4.run_raw(fmt, False, v, *args)
            assert rc == w4.OK, (fmt, v, rc)

    t0 = time.perf_counter()   # clock settling
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        run(variants[0], 8)
        torch.cuda.synchronize()
    best = {v: float("inf") for v in variants}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(rounds):
        for v in variants[r % len(variants):] + variants[:r % len(variants)]:
            run(v, 3)
            e0.record(stream)
            run(v, reps)
            e1.record(stream)
            torch.cuda.synchronize()
            best[v] = min(best[v], e0.elapsed_time(e1) * 1e3 / reps)
    return best


@pytest.mark.parametrize("fmt,shape", CASES, ids=[f"{f}-{s if isinstance(s, str) else 'x'.join(map(str, s))}"
                                                   for f, s in CASES])
def test_solver_pick_is_near_the_fastest(fmt, shape):
    if isinstance(shape, str):
        wl = synthetic.workload(shape)
        x = synthetic.make_inputs(wl, fmt=fmt)
        M, N, K, R = wl.shape
    else:
        M, N, K, R = shape
        x = synthetic.custom_inputs(M, N, K, R, seed=3000, fmt=fmt)
    _say(f"case: solver pick {fmt} M={M} N={N} K={K} R={R}")
    t = time_instances(fmt, x)
    p = w4.plan(M, N, K, R, fmt=fmt)
    pick = f"v{p['variant']}" + (f" + v{p['tail_variant']} on the last {p['tail_rows']} rows" if p["tail_variant"] >= 0 else "")
    single = {v: us for v, us in t.items() if v >= 0}
    fastest = min(single, key=single.get)
    _say("  " + ", ".join(f"v{v} {us:.1f} us" for v, us in sorted(single.items())) +
         f"; plan ({pick}) {t[-1]:.1f} us, fastest single v{fastest}")
    assert t[-1] <= 1.15 * single[fastest], (fmt, shape, pick, t)
