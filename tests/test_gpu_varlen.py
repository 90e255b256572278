"""GPU parity for rows that pack several documents (ssd_forward_varlen): the
fp64 oracle with the same document ids, where the decay is 0 at each
document start ("Transformers are SSMs", Knowl 8)."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import MaxRelErr, oracle_batch, record_parity, TOL, say, to_dev, workload

pytestmark = pytest.mark.gpu


def gpu_varlen(inp, seq, Q, state_dtype="fp32", init=None):
    d = to_dev(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], Q, state_dtype,
                         initial_state=None if init is None else init.to("cuda"), seq_idx=seq.to("cuda"))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fin.cpu().numpy().astype(np.float64)


def check(w, inp, seq, state_dtype="fp32", init=None):
    say(f"case {w.describe()} state={state_dtype} docs={int(seq[0, -1] - seq[0, 0]) + 1} "
        f"init={init is not None}")
    y, fin = gpu_varlen(inp, seq, w.chunk_size, state_dtype, init)
    f = inputs.to_float64(inp)
    y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], seq_idx=seq.numpy(),
                                       init=None if init is None else init.numpy().astype(np.float64))
    ey, ef = oracle.rel_err(y, y_ref), oracle.rel_err(fin, fin_ref)
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    t = TOL[w.dtype]
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    assert ey <= t and ef <= t, (ey, ef, t)


def test_tiny_fp32_documents():
    w = workload("tiny", batch=2, seqlen=256)
    # starts at t = 1, on a chunk boundary and one token either side of it
    check(w, inputs.generate_slow_decay(w, seed=40), inputs.generate_seq_idx(w, 40, 5, cuts=(1, 63, 64, 65)))


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("with_init", [False, True])
def test_m125_shape_ragged_documents(state_dtype, with_init):
    w = workload("m125", batch=2, seqlen=1000, nheads=4)
    init = inputs.generate_initial_state(w, seed=41) if with_init else None
    check(w, inputs.generate_slow_decay(w, seed=41), inputs.generate_seq_idx(w, 41, 6, cuts=(256, 512, 999)),
          state_dtype, init)


@pytest.mark.parametrize("Q,T", [(16, 100), (32, 100), (64, 64), (128, 300), (256, 31)])
def test_chunk_sizes_documents(Q, T):
    w = workload("m125", batch=1, seqlen=T, nheads=3, chunk_size=Q)
    check(w, inputs.generate_slow_decay(w, seed=42), inputs.generate_seq_idx(w, 42, 4, cuts=(Q,)))


def test_every_token_its_own_document():
    """Each token alone: y_t = dt_t (C_t . B_t) x_t + D x_t, the memoryless map."""
    w = workload("m125", batch=1, seqlen=300, nheads=2)
    seq = torch.arange(300, dtype=torch.int32)[None]
    check(w, inputs.generate_slow_decay(w, seed=43), seq)


def test_one_document_matches_ssd_forward():
    w = workload("m125", batch=2, seqlen=700, nheads=3)
    g = to_dev(inputs.generate(w, seed=44))
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, "bf16")
    ws = ssd.alloc_workspace(d, "cuda")
    y0, y1 = torch.empty_like(g["x"]), torch.empty_like(g["x"])
    f0 = torch.empty((2, 3, w.dstate, w.headdim), device="cuda")
    f1 = torch.empty_like(f0)
    seq = torch.tensor([[3], [9]], dtype=torch.int32, device="cuda").expand(2, 700).contiguous()
    ssd.ssd_forward(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y0, f0, ws, ws.numel())
    ssd.ssd_forward_varlen(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, seq, y1, f1, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.allclose(y0.float(), y1.float(), rtol=0, atol=1e-2 * y0.float().abs().max().item())
    assert torch.allclose(f0, f1, rtol=1e-5, atol=1e-5 * f0.abs().max().item())


@pytest.mark.parametrize("name", ["m2p7", "nsweep256"])
def test_fullsize_documents_whole_output(name):
    """The full workload with eight documents per row, in the configuration the
    forward runs at that size, against the oracle with the same ids over the
    whole output (every batch element and head)."""
    w = inputs.WORKLOADS[name]
    say(f"fullsize varlen {name} {w.describe()}")
    inp = inputs.generate(w, seed=0)
    seq = inputs.generate_seq_idx(w, 45, 8, cuts=(w.chunk_size, 2 * w.chunk_size + 1))
    y, fin = ssd.forward(*(inp[k].to("cuda") for k in ("x", "dt", "A", "B", "C", "D")), w.chunk_size,
                         seq_idx=seq.to("cuda"))
    torch.cuda.synchronize()
    ey, ef = MaxRelErr(), MaxRelErr()
    for b in range(w.batch):
        y_ref, fin_ref = oracle_batch(inp, b, seq_idx=seq.numpy())
        ey.add(y[b].float().cpu().numpy(), y_ref[0])
        ef.add(fin[b].cpu().numpy(), fin_ref[0])
    record_parity("varlen", name, "bf16", ey.value(), ef.value(), TOL[w.dtype])
    assert ey.value() <= TOL[w.dtype] and ef.value() <= TOL[w.dtype]


def check_gated(w, inp, seq, z, state_dtype="fp32", init=None):
    """ssd_forward_varlen_gated against the oracle's recurrence with the same
    ids, then its SiLU gate ("Transformers are SSMs", Knowl 6 and Knowl 8)."""
    say(f"case {w.describe()} gated docs state={state_dtype} init={init is not None}")
    d = to_dev(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_size, state_dtype,
                         initial_state=None if init is None else init.to("cuda"), seq_idx=seq.to("cuda"),
                         z=z.to("cuda"))
    torch.cuda.synchronize()
    f = inputs.to_float64(inp)
    y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], seq_idx=seq.numpy(),
                                       init=None if init is None else init.numpy().astype(np.float64))
    y_ref = oracle.silu_gate(y_ref, z.float().numpy())
    ey = oracle.rel_err(y.float().cpu().numpy(), y_ref)
    ef = oracle.rel_err(fin.cpu().numpy(), fin_ref)
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    t = TOL[w.dtype]
    assert ey <= t and ef <= t, (ey, ef, t)


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("with_init", [False, True])
def test_gated_documents_ragged(state_dtype, with_init):
    w = workload("m125", batch=2, seqlen=1000, nheads=4)
    init = inputs.generate_initial_state(w, seed=46) if with_init else None
    check_gated(w, inputs.generate_slow_decay(w, seed=46), inputs.generate_seq_idx(w, 46, 6, cuts=(256, 512, 999)),
                inputs.generate_gate(w, seed=46), state_dtype, init)


@pytest.mark.parametrize("Q,T", [(16, 100), (64, 200), (256, 300)])
def test_gated_documents_chunk_sizes(Q, T):
    w = workload("m125", batch=1, seqlen=T, nheads=3, chunk_size=Q)
    check_gated(w, inputs.generate_slow_decay(w, seed=47), inputs.generate_seq_idx(w, 47, 4, cuts=(Q,)),
                inputs.generate_gate(w, seed=47))


def test_gated_documents_fp32_inputs():
    w = workload("tiny", batch=2, seqlen=256)
    check_gated(w, inputs.generate_slow_decay(w, seed=48), inputs.generate_seq_idx(w, 48, 5, cuts=(1, 64)),
                inputs.generate_gate(w, seed=48))


def test_gated_documents_match_gated_forward_on_one_document():
    """One document per row: the same output as ssd_forward_gated."""
    w = workload("m125", batch=2, seqlen=700, nheads=3)
    g = to_dev(inputs.generate(w, seed=49))
    z = inputs.generate_gate(w, seed=49).cuda()
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, "bf16")
    ws = ssd.alloc_workspace(d, "cuda")
    y0, y1 = torch.empty_like(g["x"]), torch.empty_like(g["x"])
    f0 = torch.empty((2, 3, w.dstate, w.headdim), device="cuda")
    f1 = torch.empty_like(f0)
    seq = torch.tensor([[3], [9]], dtype=torch.int32, device="cuda").expand(2, 700).contiguous()
    ssd.ssd_forward_gated(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, z, y0, f0, ws, ws.numel())
    ssd.ssd_forward_varlen_gated(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, seq, z, y1, f1, ws,
                                 ws.numel())
    torch.cuda.synchronize()
    assert torch.allclose(y0.float(), y1.float(), rtol=0, atol=1e-2 * y0.float().abs().max().item())
    assert torch.allclose(f0, f1, rtol=1e-5, atol=1e-5 * f0.abs().max().item())


def test_fullsize_gated_documents_whole_output():
    """The 2.7B-layer workload with eight documents per row and the gate, in
    the configuration the forward runs at that size, against the oracle's
    recurrence with the same ids and its gate, over the whole output."""
    w = inputs.WORKLOADS["m2p7"]
    say(f"fullsize gated varlen m2p7 {w.describe()}")
    inp = inputs.generate(w, seed=0)
    seq = inputs.generate_seq_idx(w, 45, 8, cuts=(w.chunk_size, 2 * w.chunk_size + 1))
    z = inputs.generate_gate(w, seed=1)
    y, fin = ssd.forward(*(inp[k].to("cuda") for k in ("x", "dt", "A", "B", "C", "D")), w.chunk_size,
                         seq_idx=seq.to("cuda"), z=z.to("cuda"))
    torch.cuda.synchronize()
    ey, ef = MaxRelErr(), MaxRelErr()
    zf = z.float().numpy()
    for b in range(w.batch):
        y_ref, fin_ref = oracle_batch(inp, b, seq_idx=seq.numpy())
        ey.add(y[b].float().cpu().numpy(), oracle.silu_gate(y_ref[0], zf[b]))
        ef.add(fin[b].cpu().numpy(), fin_ref[0])
    record_parity("varlen+gate", "m2p7", "bf16", ey.value(), ef.value(), TOL[w.dtype])
    assert ey.value() <= TOL[w.dtype] and ef.value() <= TOL[w.dtype]
