"""GPU parity for the fused output gate (ssd_forward_gated: y * silu(z) in the
chunk scan's epilogue) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import TOL, say, to_dev, workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,state_dtype,with_init", [
    ("tiny", {}, "fp32", False),
    ("tiny", dict(batch=2, seqlen=333, nheads=3, headdim=64, dstate=128, chunk_size=128), "fp32", True),
    ("m125", dict(batch=2, seqlen=1000, nheads=4), "bf16", False),
    ("m125", dict(batch=1, seqlen=520, nheads=3, headdim=16, dstate=256, chunk_size=64), "fp32", True),
    ("m125", dict(batch=1, seqlen=200, nheads=2, chunk_size=16), "bf16", True),
])
def test_gated_forward(name, kw, state_dtype, with_init):
    w = workload(name, **kw)
    inp = inputs.generate_slow_decay(w, seed=50)
    z = inputs.generate_gate(w, seed=50)
    init = inputs.generate_initial_state(w, seed=50) if with_init else None
    say(f"gated {w.describe()} state={state_dtype} init={with_init}")
    g = to_dev(inp)
    y, fin = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], w.chunk_size, state_dtype,
                         initial_state=None if init is None else init.to("cuda"), z=z.to("cuda"))
    torch.cuda.synchronize()
    f = inputs.to_float64(inp)
    y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"],
                                       init=None if init is None else init.numpy().astype(np.float64))
    yg_ref = oracle.silu_gate(y_ref, z.float().numpy().astype(np.float64))
    ey = oracle.rel_err(y.float().cpu().numpy().astype(np.float64), yg_ref)
    ef = oracle.rel_err(fin.cpu().numpy().astype(np.float64), fin_ref)
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]


def test_gate_changes_only_the_output():
    """The final state is the ungated forward's, bitwise; the gated y equals
    the ungated y times silu(z) to the output type's rounding."""
    w = workload("m125", batch=1, seqlen=700, nheads=3)
    g = to_dev(inputs.generate(w, seed=51))
    z = inputs.generate_gate(w, seed=51).to("cuda")
    y0, f0 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], w.chunk_size)
    y1, f1 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], w.chunk_size, z=z)
    torch.cuda.synchronize()
    assert torch.equal(f0, f1)
    ref = y0.float() * torch.nn.functional.silu(z.float())
    err = (y1.float() - ref).abs().max().item() / ref.abs().max().item()
    say(f"gated vs ungated*silu: {err:.3e}")
    assert err <= 1e-2
