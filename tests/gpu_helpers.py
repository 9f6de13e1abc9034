"""Helpers shared by the GPU parity tests: device upload, row sampling and the
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


def assert_parity(got, y, T, what, dtype="bf16"):
    res = ref.check_output(got, y, T, dtype)
    _say(f"  {what}: max err/bound {res['max_ratio']:.3g}, failures {res['n_fail']}")
    assert res["ok"], (what, res)


def _sample_rows(M, block_m, rng):
    rows = set(range(0, min(M, 40)))                          # first tile head
    rows |= set(range(max(0, M - 40), M))                     # last (ragged) rows
    for t in range(0, M, block_m):                            # tile boundaries
        rows |= {t, min(M - 1, t + block_m - 1)}
    rows |= set(rng.choice(M, size=min(M, 64), replace=False).tolist())
    return np.array(sorted(rows))
