"""GPU parity for a given initial state (ssd_forward_init and the stage entry
points ssd_state_passing_init / ssd_chunk_scan_init) against the fp64 oracle
started from the same state."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import TOL, say, to_dev, workload

pytestmark = pytest.mark.gpu


def gpu_forward_init(inp, init, Q, state_dtype="fp32"):
    d = to_dev(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], Q, state_dtype,
                         initial_state=init.to("cuda"))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fin.cpu().numpy().astype(np.float64)


def oracle_init(inp, init):
    f = inputs.to_float64(inp)
    return oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"],
                             init=init.numpy().astype(np.float64))


def check(w, inp, init, state_dtype="fp32"):
    say(f"case {w.describe()} state={state_dtype} with initial state")
    y, fin = gpu_forward_init(inp, init, w.chunk_size, state_dtype)
    y_ref, fin_ref = oracle_init(inp, init)
    ey, ef = oracle.rel_err(y, y_ref), oracle.rel_err(fin, fin_ref)
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    t = TOL[w.dtype]
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    assert ey <= t and ef <= t, (ey, ef, t)


def test_tiny_fp32_with_initial_state():
    w = workload("tiny")
    check(w, inputs.generate_slow_decay(w, seed=30), inputs.generate_initial_state(w, seed=30))


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_m125_shape_ragged_with_initial_state(state_dtype):
    w = workload("m125", batch=2, seqlen=1000, nheads=4)
    check(w, inputs.generate_slow_decay(w, seed=31), inputs.generate_initial_state(w, seed=31), state_dtype)


@pytest.mark.parametrize("Q,T", [(16, 100), (32, 100), (64, 64), (128, 300), (256, 31)])
def test_chunk_sizes_with_initial_state(Q, T):
    w = workload("m125", batch=1, seqlen=T, nheads=3, chunk_size=Q)
    check(w, inputs.generate_slow_decay(w, seed=32), inputs.generate_initial_state(w, seed=32))


def test_initial_state_only_response():
    """x = 0: y is the initial state's free decay read out by C (every other
    term vanishes), so the first chunk's carried-state term is checked alone."""
    w = workload("tiny", batch=2, seqlen=200, nheads=2)
    inp = inputs.generate_slow_decay(w, seed=33)
    inp["x"] = torch.zeros_like(inp["x"])
    check(w, inp, inputs.generate_initial_state(w, seed=33))


def test_null_initial_state_is_ssd_forward():
    w = workload("m125", batch=1, seqlen=700, nheads=3)
    g = to_dev(inputs.generate(w, seed=34))
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, "bf16")
    ws = ssd.alloc_workspace(d, "cuda")
    y0, y1 = torch.empty_like(g["x"]), torch.empty_like(g["x"])
    f0 = torch.empty((1, 3, w.dstate, w.headdim), device="cuda")
    f1 = torch.empty_like(f0)
    ssd.ssd_forward(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y0, f0, ws, ws.numel())
    ssd.ssd_forward_init(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, y1, f1, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_resume_from_prefix_final_state(state_dtype):
    """Run [0, T1), then [T1, T) from its final state: the second part matches
    the oracle's full run over [0, T)."""
    w = workload("m125", batch=2, seqlen=900, nheads=3)
    inp = inputs.generate_slow_decay(w, seed=35)
    T1 = 333
    first = {k: (v[:, :T1].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    rest = {k: (v[:, T1:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    d1 = to_dev(first)
    _, f1 = ssd.forward(d1["x"], d1["dt"], d1["A"], d1["B"], d1["C"], d1["D"], w.chunk_size, state_dtype)
    d2 = to_dev(rest)
    y2, f2 = ssd.forward(d2["x"], d2["dt"], d2["A"], d2["B"], d2["C"], d2["D"], w.chunk_size, state_dtype,
                         initial_state=f1)
    torch.cuda.synchronize()
    f = inputs.to_float64(inp)
    y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"])
    ey = oracle.rel_err(y2.float().cpu().numpy().astype(np.float64), y_ref[:, T1:])
    ef = oracle.rel_err(f2.cpu().numpy().astype(np.float64), fin_ref)
    say(f"resume at {T1}: err_y={ey:.3e} err_final={ef:.3e}")
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]


def test_stage_entry_points_with_initial_state():
    """cumsum+state, state passing and chunk scan from an initial state, one by
    one, give bitwise what ssd_forward_init gives."""
    w = workload("m125", batch=1, seqlen=600, nheads=4)
    g = to_dev(inputs.generate_slow_decay(w, seed=36))
    init = inputs.generate_initial_state(w, seed=36).to("cuda")
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, "bf16")
    b, H, P, N, nc, Q = d.batch, d.nheads, d.headdim, d.dstate, d.nchunks, d.chunk_size
    cs = torch.empty((b, H, nc, Q), device="cuda")
    states = torch.empty((b, nc, H, P, N), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((b, H, N, P), device="cuda")
    y = torch.empty_like(g["x"])
    ssd.ssd_chunk_cumsum_state(d, g["x"], g["dt"], g["A"], g["B"], cs, states)
    ssd.ssd_state_passing_init(d, cs, states, init, fin)
    ssd.ssd_chunk_scan_init(d, g["x"], g["dt"], g["B"], g["C"], g["D"], cs, states, y)
    y2, fin2 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], w.chunk_size, "bf16",
                           initial_state=init)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(fin, fin2)
    # h_0 as stored for the chunk scan is the initial state ([P][N], bf16)
    h0 = states[:, 0].float().transpose(-1, -2)
    assert torch.equal(h0, init.to(torch.bfloat16).float())


def test_empty_sequence_copies_initial_state():
    w = workload("m125", batch=2, seqlen=0, nheads=2)
    init = inputs.generate_initial_state(w, seed=37).to("cuda")
    d = ssd.make_dims(2, 0, 2, w.headdim, w.dstate, 1, w.chunk_size, "bf16", "bf16")
    fin = torch.full_like(init, float("nan"))
    ssd.ssd_forward_init(d, None, None, None, None, None, None, init, None, fin, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)
