"""Shared helpers for the GPU parity tests (test infrastructure)."""
import numpy as np
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs

# Tolerances on max|dy| / max|y| (and the same for the final state): 1e-4 for
# fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation.
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def to_dev(inp, device="cuda"):
    return {k: v.to(device) for k, v in inp.items()}


def gpu_forward(inp, Q, state_dtype="fp32"):
    d = to_dev(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], Q, state_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fin.cpu().numpy().astype(np.float64)


def oracle_forward(inp, snap_every=0):
    f = inputs.to_float64(inp)
    return oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], snap_every=snap_every)


def workload(name, **kw):
    return inputs.WORKLOADS[name].replace(**kw) if kw else inputs.WORKLOADS[name]


def say(msg):
    print(msg, flush=True)
