"""GPU parity for the decoding step ssd_step against the fp64 oracle: one token
of the recurrence from a given state, and many steps continuing a prompt run
through ssd_forward."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import TOL, say, to_dev, workload

pytestmark = pytest.mark.gpu


def token(inp, t):
    """Token t of a generated sequence, as the step's [b,H,P] / [b,H] / [b,G,N] inputs."""
    return {k: (v[:, t].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}


def oracle_steps(inp, init):
    f = inputs.to_float64(inp)
    return oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"],
                             init=init.astype(np.float64))


@pytest.mark.parametrize("name,P,N,H,G", [("tiny", 16, 16, 4, 1), ("m125", 64, 128, 8, 1),
                                          ("m125", 32, 64, 6, 2), ("m125", 128, 256, 4, 4),
                                          ("tiny", 64, 128, 3, 3)])
def test_one_step(name, P, N, H, G):
    w = workload(name, batch=2, seqlen=1, nheads=H, headdim=P, dstate=N, ngroups=G)
    inp = inputs.generate_slow_decay(w, seed=40)
    init = inputs.generate_initial_state(w, seed=40)
    say(f"step {w.describe()}")
    g = to_dev(token(inp, 0))
    state = init.to("cuda").clone()
    y = ssd.step(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], state)
    torch.cuda.synchronize()
    y_ref, st_ref = oracle_steps(inp, init.numpy())
    ey = oracle.rel_err(y.float().cpu().numpy().astype(np.float64), y_ref[:, 0])
    es = oracle.rel_err(state.cpu().numpy().astype(np.float64), st_ref)
    say(f"  err_y={ey:.3e} err_state={es:.3e}")
    # one step rounds only its own products: fp32 accuracy for the state,
    # the output type's for y
    assert es <= 1e-5
    assert ey <= (1e-5 if w.dtype == "fp32" else 8e-3)


@pytest.mark.parametrize("name", ["tiny", "m125"])
def test_steps_continue_a_prompt(name):
    """A prompt of 300 tokens through ssd_forward, then 60 tokens one at a time
    from its final state: every step's y and the last state match the oracle's
    run over all 360 tokens."""
    w = workload(name, batch=2, seqlen=360, nheads=3)
    inp = inputs.generate_slow_decay(w, seed=41)
    T1 = 300
    prompt = {k: (v[:, :T1].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    d = to_dev(prompt)
    _, state = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_size)
    ys = []
    for t in range(T1, 360):
        g = to_dev(token(inp, t))
        ys.append(ssd.step(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], state))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1).float().cpu().numpy().astype(np.float64)
    f = inputs.to_float64(inp)
    y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"])
    ey = oracle.rel_err(y, y_ref[:, T1:])
    es = oracle.rel_err(state.cpu().numpy().astype(np.float64), fin_ref)
    say(f"{name}: 60 steps after a {T1}-token prompt: err_y={ey:.3e} err_state={es:.3e}")
    assert ey <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_zero_batch_is_a_no_op():
    d = ssd.make_dims(0, 1, 2, 64, 128, 1, 32, "bf16", "fp32")
    ssd.ssd_step(d, None, None, None, None, None, None, None, None, stream=0)
