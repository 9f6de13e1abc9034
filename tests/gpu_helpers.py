"""Helpers shared by the GPU parity tests: device upload, the full oracle, row
sampling (only for outputs too large to hold twice on the host) and the
tolerance check (oracle.check_output)."""
import sys

import numpy as np
import torch

import oracle.w4a4_ref as ref

DEV = "cuda:0"
ARGS = ("act", "ascales", "wgt", "wscales", "wcscale", "bias", "lora_act_in", "lora_up")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x):
    d = {}
    for k in ("act", "ascales", "wgt", "wscales"):
        d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).to(DEV)
    d["wcscale"] = torch.from_numpy(np.ascontiguousarray(x["wcscale"])).to(DEV)
    d["bias"] = torch.from_numpy(np.ascontiguousarray(x["bias"])).to(DEV)
    half = torch.float16 if x.get("dtype", "bf16") == "f16" else torch.bfloat16
    if x["R"] > 0:
        for k in ("lora_act_in", "lora_up"):
            t = torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16))
            d[k] = t.view(half).to(DEV)
    else:
        d["lora_act_in"] = d["lora_up"] = None
    return d


def full_reference(x, fmt="nvfp4"):
    """(y, T) of the oracle over every output element."""
    a = [x[k] for k in ARGS]
    dt = x.get("dtype", "bf16")
    if fmt == "mxfp4":
        return ref.gemm_mxfp4_ref(*a, dtype=dt), ref.term_magnitude_mx(*a, dtype=dt)
    return ref.gemm_w4a4_ref(*a, dtype=dt), ref.term_magnitude(*a, dtype=dt)


def assert_parity(got, y, T, what, dtype="bf16"):
    res = ref.check_output(got, y, T, dtype)
    _say(f"  {what}: {got.size} elements, max err/bound {res['max_ratio']:.3g}, "
         f"failures {res['n_fail']}")
    assert res["ok"], (what, res)
