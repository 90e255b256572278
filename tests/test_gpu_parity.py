"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Sizes here are ones the oracle finishes in seconds but that still span several
32-row tiles, several chunks and a ragged last chunk. Full-size workloads are
checked over their whole output in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import TOL, gpu_forward, oracle_forward, say, to_dev, workload

pytestmark = pytest.mark.gpu


def check(w, inp, state_dtype="fp32", tol=None):
    say(f"case {w.describe()} state={state_dtype}")
    y, fin = gpu_forward(inp, w.chunk_size, state_dtype)
    y_ref, fin_ref = oracle_forward(inp)
    ey, ef = oracle.rel_err(y, y_ref), oracle.rel_err(fin, fin_ref)
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    t = tol or TOL[w.dtype]
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    assert ey <= t, f"y error {ey} > {t}"
    assert ef <= t, f"final state error {ef} > {t}"
    return ey, ef


def test_tiny_fp32_full():
    """The tiny fp32 workload at its full size: b1 T256 H2 P16 N16 Q64."""
    w = workload("tiny")
    check(w, inputs.generate(w))


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_m125_shape_ragged(state_dtype):
    """125M-layer head shape (P64 N128 Q256) with a ragged last chunk (T=1000)."""
    w = workload("m125", batch=2, seqlen=1000, nheads=4)
    check(w, inputs.generate(w, seed=1), state_dtype)


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_slow_decay_inter_chunk_path(state_dtype):
    """|A| in [1e-3, 1e-1]: the state carried between chunks dominates y."""
    w = workload("m125", batch=1, seqlen=1024, nheads=3)
    check(w, inputs.generate_slow_decay(w, seed=2), state_dtype)


@pytest.mark.parametrize("Q", [16, 32, 64, 128, 256])
def test_chunk_sizes(Q):
    w = workload("m125", batch=1, seqlen=600, nheads=2, chunk_size=Q)
    check(w, inputs.generate_slow_decay(w, seed=3))


@pytest.mark.parametrize("T", [16, 17, 100, 257])
@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_chunk_size_16(T, state_dtype):
    """Q = 16 ("Transformers are SSMs", Knowl 2 takes Q = N = P; N = P = 16 is
    the tiny shape): each chunk fills half of a 32-token tile, the other half
    masked like the tail of a short last chunk; ragged T included."""
    w = workload("m125", batch=2, seqlen=T, nheads=4, headdim=64, dstate=128, chunk_size=16)
    check(w, inputs.generate_slow_decay(w, seed=31), state_dtype)


def test_chunk_size_16_tiny_fp32():
    """The tiny fp32 shape with Q = N = P = 16."""
    w = workload("tiny", chunk_size=16)
    check(w, inputs.generate(w, seed=32))


@pytest.mark.parametrize("P,N,state", [(16, 16, "fp32"), (32, 64, "fp32"), (64, 16, "fp32"), (64, 256, "fp32"),
                                         (128, 128, "fp32"), (128, 256, "bf16"), (16, 256, "fp32")])
def test_head_and_state_dims(P, N, state):
    w = workload("m125", batch=1, seqlen=520, nheads=3, headdim=P, dstate=N)
    check(w, inputs.generate_slow_decay(w, seed=4), state)


@pytest.mark.parametrize("H,G", [(6, 2), (6, 6), (24, 8)])
def test_group_patterns(H, G):
    """Knowl 7: multi-input (G=1, other tests), grouped (1<G<H) and multi-head (G=H)."""
    w = workload("m125", batch=2, seqlen=300, nheads=H, ngroups=G)
    check(w, inputs.generate_slow_decay(w, seed=5))


@pytest.mark.parametrize("P,N,state,Q", [(128, 256, "fp32", 64), (128, 256, "bf16", 128), (64, 256, "fp32", 256)])
def test_large_state_tiles(P, N, state, Q):
    """Head and state sizes whose LDS tiles leave little room: the chunk scan
    falls back to single buffers and, at the largest, to C B^T in registers."""
    w = workload("m125", batch=1, seqlen=2 * Q + 40, nheads=3, headdim=P, dstate=N, chunk_size=Q)
    check(w, inputs.generate_slow_decay(w, seed=12), state)


@pytest.mark.parametrize("P,N,Q", [(16, 16, 64), (64, 128, 128), (32, 32, 32), (64, 64, 256), (16, 16, 16)])
def test_fp32_inputs(P, N, Q):
    w = workload("tiny", batch=2, seqlen=333, nheads=3, headdim=P, dstate=N, chunk_size=Q)
    check(w, inputs.generate_slow_decay(w, seed=6))


@pytest.mark.parametrize("T", [1, 31, 32, 33, 255, 257])
def test_short_and_boundary_lengths(T):
    w = workload("m125", batch=2, seqlen=T, nheads=2)
    check(w, inputs.generate_slow_decay(w, seed=7))


def test_no_decay_linear_attention():
    """A = 0 (a = 1 everywhere): nothing decays, every path carries full weight."""
    w = workload("m125", batch=1, seqlen=700, nheads=2)
    inp = inputs.generate(w, seed=8)
    inp["A"] = torch.zeros_like(inp["A"])
    check(w, inp)


def test_full_decay_memoryless():
    """dt*A <= -800: a = 0, y_t = dt_t (C_t.B_t) x_t + D x_t."""
    w = workload("tiny", batch=1, seqlen=200, nheads=2)
    inp = inputs.generate(w, seed=9)
    inp["dt"] = torch.full_like(inp["dt"], 50.0)
    inp["A"] = torch.full_like(inp["A"], -20.0)
    check(w, inp)


def test_empty_inputs():
    w = workload("m125", batch=2, seqlen=64, nheads=2)
    inp = to_dev(inputs.generate(w))
    # seqlen 0: final state is zero, nothing else touched
    x0 = inp["x"][:, :0].contiguous()
    B0 = inp["B"][:, :0].contiguous()
    y, fin = ssd.forward(x0, inp["dt"][:, :0].contiguous(), inp["A"], B0, inp["C"][:, :0].contiguous(),
                         inp["D"], 256)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.all(fin == 0)
    # batch 0
    y, fin = ssd.forward(inp["x"][:0], inp["dt"][:0], inp["A"], inp["B"][:0], inp["C"][:0], inp["D"], 256)
    torch.cuda.synchronize()
    assert y.numel() == 0 and fin.numel() == 0


def test_deterministic_and_fully_written():
    """Two runs agree bitwise, and no output or intermediate is left unwritten
    (outputs and workspace prefilled with NaN)."""
    w = workload("m125", batch=2, seqlen=777, nheads=4)
    inp = to_dev(inputs.generate(w, seed=10))
    d = ssd.dims_of(inp["x"], inp["B"], w.chunk_size)
    outs = []
    for _ in range(2):
        ws = torch.full((ssd.ssd_workspace_size(d),), 255, dtype=torch.uint8, device="cuda")
        y = torch.full_like(inp["x"], float("nan"))
        fin = torch.full((w.batch, w.nheads, w.dstate, w.headdim), float("nan"), device="cuda")
        ssd.ssd_forward(d, inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], y, fin, ws,
                        ws.numel())
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
        outs.append((y.clone(), fin.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T,Q", [(900, 256), (16384, 256), (900, 16)])
def test_stage_parity(state_dtype, T, Q):
    """Each stage against its fp64 counterpart: cs against the block algorithm's
    prefix sums, S against its chunk states, h_in against the recurrence's state
    at every chunk boundary, final and y against the recurrence; T = 16384 is a
    chain of 64 chunk states on slow-decay rows, where rounding that compounded
    along the chain would show."""
    w = workload("m125", batch=2 if T < 4096 else 1, seqlen=T, nheads=3, ngroups=1, chunk_size=Q)
    inp = inputs.generate_slow_decay(w, seed=11)
    say(f"stage case {w.describe()} state={state_dtype}")
    dev = to_dev(inp)
    out = ssd.stages(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], w.chunk_size, state_dtype)
    torch.cuda.synchronize()
    f = inputs.to_float64(inp)
    ref = oracle.chunked(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], Q=w.chunk_size)
    y_ref, fin_ref, snaps = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"],
                                              snap_every=w.chunk_size)
    cs = out["cs"].cpu().numpy().astype(np.float64)
    valid = ~np.isnan(ref["cs"])
    assert oracle.rel_err(cs[valid], ref["cs"][valid]) < 1e-5
    # padding positions of the ragged chunk repeat the chunk's last value
    last = w.seqlen - (w.nchunks - 1) * w.chunk_size
    assert np.all(cs[:, :, -1, last:] == cs[:, :, -1, last - 1: last])
    tol = TOL[w.dtype]
    S = out["S"].float().cpu().numpy().astype(np.float64).transpose(0, 1, 2, 4, 3)   # -> [b,nc,H,N,P]
    assert oracle.rel_err(S, ref["S"]) < tol
    h_in = out["h_in"].float().cpu().numpy().astype(np.float64).transpose(0, 1, 2, 4, 3)
    assert oracle.rel_err(h_in, snaps) < tol
    assert oracle.rel_err(out["final"].cpu().numpy(), fin_ref) < tol
    assert oracle.rel_err(out["y"].float().cpu().numpy(), y_ref) < tol


@pytest.mark.parametrize("T", [1000, 512])
def test_forward_matches_stage_entry_points(T):
    """ssd_forward fuses the in-chunk cumulative decay into its chunk-state
    launch; the result must be bitwise that of the four stage entry points."""
    w = workload("m125", batch=2, seqlen=T, nheads=6, ngroups=2)
    dev = to_dev(inputs.generate_slow_decay(w, seed=13))
    say(f"fused-vs-stages case {w.describe()}")
    for st in ("fp32", "bf16"):
        y, fin = ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], w.chunk_size, st)
        out = ssd.stages(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], w.chunk_size, st)
        d = ssd.dims_of(dev["x"], dev["B"], w.chunk_size, st)
        cs = torch.full_like(out["cs"], float("nan"))
        S = torch.full_like(out["S"], float("nan"))
        ssd.ssd_chunk_cumsum_state(d, dev["x"], dev["dt"], dev["A"], dev["B"], cs, S)
        torch.cuda.synchronize()
        assert torch.equal(y, out["y"]) and torch.equal(fin, out["final"])
        assert torch.equal(cs, out["cs"]) and torch.equal(S, out["S"])


def test_prepared_call_matches_the_checked_call():
    """A call repeated through ssd.prepared gives bitwise what the checked
    wrapper gives."""
    w = workload("m125", batch=2, seqlen=600, nheads=4)
    g = to_dev(inputs.generate(w, seed=61))
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, "bf16")
    ws = ssd.alloc_workspace(d, "cuda")
    y0, y1 = torch.empty_like(g["x"]), torch.full_like(g["x"], float("nan"))
    f0 = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), device="cuda")
    f1 = torch.full_like(f0, float("nan"))
    ssd.ssd_forward(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y0, f0, ws, ws.numel())
    call = ssd.prepared(ssd.ssd_forward, d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y1, f1, ws, ws.numel())
    call()
    call()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
