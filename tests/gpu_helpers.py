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


# ---- whole-output error figures -------------------------------------------------

# (what, workload, state storage, err_y, err_final, tolerance) of every
# whole-output comparison this session, printed in the terminal summary
PARITY_RECORDS = []


class MaxRelErr:
    """max|got - ref| / max|ref| accumulated over pieces of one output (the
    pieces together cover it), so the figure is that of the whole output."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if ref.size:
            self.num = max(self.num, float(np.max(np.abs(got - ref))))
            self.den = max(self.den, float(np.max(np.abs(ref))))

    def value(self) -> float:
        return self.num / self.den if self.den > 0 else self.num


def batch_slice(inp, b):
    """Inputs of batch element b alone (A and D are per head, shared)."""
    return {k: (v[b:b + 1] if v.dim() > 1 else v) for k, v in inp.items()}


def oracle_batch(inp, b, seq_idx=None, init=None):
    """The oracle on batch element b (every head): rows are independent, so this
    is the whole output's row b. Returns y [1,T,H,P], final [1,H,N,P]."""
    f = inputs.to_float64(batch_slice(inp, b))
    seq = None if seq_idx is None else np.asarray(seq_idx[b:b + 1])
    ini = None if init is None else np.asarray(init[b:b + 1], dtype=np.float64)
    return oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], seq_idx=seq, init=ini)


def record_parity(what, name, state_dtype, err_y, err_final, tol):
    PARITY_RECORDS.append((what, name, state_dtype, err_y, err_final, tol))
    ef = "-" if err_final is None else f"{err_final:.3e}"
    say(f"PARITY {what} {name} states={state_dtype}: err_y={err_y:.3e} err_final={ef} (tol {tol:g})")
