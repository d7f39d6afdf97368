"""Helpers for the GPU tests: move seeded inputs to the device and back."""
import os
import sys

import numpy as np
import torch

import ssd_inputs as si


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(arr, dtype):
    """numpy array (float32, or uint16 bf16 bits) -> contiguous cuda tensor."""
    if dtype == si.BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to("cuda")


def host_f64(t):
    """cuda tensor (bf16 or f32) -> float64 numpy (exact widening)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def upload_fwd(d):
    dt = d["shape"].dtype
    out = {k: dev_tensor(d[k], dt) for k in ("X", "B", "C")}
    out["a"] = dev_tensor(d["a"], si.F32)
    if "S0" in d:
        out["S0"] = dev_tensor(d["S0"], si.F32)
    return out


def widen_fwd(d):
    dt = d["shape"].dtype
    out = {k: si.widen(d[k], dt) for k in ("X", "B", "C")}
    out["a"] = d["a"].astype(np.float64)
    if "S0" in d:
        out["S0"] = d["S0"].astype(np.float64)
    return out


def oracle_threads():
    return max(1, min(16, os.cpu_count() or 1))
