"""GPU parity for the normalisation after the gate (ssd_gated_rmsnorm,
"Transformers are SSMs", Knowl 6) against the fp64 oracle's gated_rmsnorm on
the same input bits, alone and after the gated forward."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import MaxRelErr, record_parity, TOL, say, to_dev, workload

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("groups", [1, 2, 8])
@pytest.mark.parametrize("gate", [False, True])
def test_norm_alone(dtype, groups, gate):
    g = torch.Generator().manual_seed(70 + groups)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    b, T, H, P = 2, 37, 6, 64
    y = torch.randn((b, T, H, P), generator=g).to(tdt)
    z = torch.randn((b, T, H, P), generator=g).to(tdt) if gate else None
    w = torch.randn(H * P, generator=g)
    say(f"norm dtype={dtype} groups={groups} gate={gate}")
    out = ssd.gated_rmsnorm(y.cuda(), None if z is None else z.cuda(), w.cuda(), 1e-5, groups)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(_f64(y), None if z is None else _f64(z), w.numpy(), 1e-5, groups)
    e = oracle.rel_err(_f64(out), ref)
    say(f"  err={e:.3e}")
    assert e <= TOL[dtype]


def test_norm_in_place_matches_out_of_place():
    g = torch.Generator().manual_seed(75)
    y = torch.randn((3, 50, 4, 32), generator=g).to(torch.bfloat16).cuda()
    w = torch.randn(128, generator=g).cuda()
    a = ssd.gated_rmsnorm(y, None, w, 1e-6, 4)
    yy = y.clone()
    ssd.gated_rmsnorm(yy, None, w, 1e-6, 4, out=yy)
    torch.cuda.synchronize()
    assert torch.equal(a, yy)


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_gated_forward_then_norm(state_dtype):
    """ssd_forward_gated, then the norm in place: the block's output before
    the out-projection, against recurrence -> gate -> norm in fp64."""
    w = workload("m125", batch=2, seqlen=600, nheads=4)
    inp = inputs.generate_slow_decay(w, seed=76)
    z = inputs.generate_gate(w, seed=76)
    wt = torch.randn(w.nheads * w.headdim, generator=torch.Generator().manual_seed(76))
    say(f"case {w.describe()} gated + norm, state={state_dtype}")
    d = to_dev(inp)
    y, _ = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_size, state_dtype, z=z.cuda())
    ssd.gated_rmsnorm(y, None, wt.cuda(), 1e-5, 1, out=y)
    torch.cuda.synchronize()
    f = inputs.to_float64(inp)
    y_ref, _ = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"])
    ref = oracle.gated_rmsnorm(y_ref, _f64(z), wt.numpy(), 1e-5, 1)
    e = oracle.rel_err(_f64(y), ref)
    say(f"  err={e:.3e}")
    assert e <= TOL[w.dtype]


def test_norm_full_size_layer_shape():
    """The headline layer shape (b=8, T=4096, 80 heads of 64): the norm of the
    gated forward's output, against the oracle's norm of the same bits, over
    every token."""
    w = inputs.WORKLOADS["m2p7"]
    inp = inputs.generate(w, seed=0)
    z = inputs.generate_gate(w, seed=1).cuda()
    wt = torch.randn(w.nheads * w.headdim, generator=torch.Generator().manual_seed(77)).cuda()
    d = to_dev(inp)
    y, _ = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_size, z=z)
    out = ssd.gated_rmsnorm(y, None, wt, 1e-5, 1)
    torch.cuda.synchronize()
    e = MaxRelErr()
    wn = wt.cpu().numpy()
    for b in range(w.batch):
        ref = oracle.gated_rmsnorm(_f64(y[b:b + 1]), None, wn, 1e-5, 1)
        e.add(_f64(out[b:b + 1]), ref)
    record_parity("rmsnorm", "m2p7", "bf16", e.value(), None, TOL[w.dtype])
    assert e.value() <= TOL[w.dtype]


def test_norm_streaming_gate_in_place():
    """A pass over more than the 256 MiB last-level cache (y, z and out of
    b=3, T=4096, 80 heads of 64, bf16: 377 MB) takes the non-temporal loads
    and stores: gated, in place and out of place, against the oracle over
    every token."""
    g = torch.Generator().manual_seed(78)
    shape = (3, 4096, 80, 64)
    y = torch.randn(shape, generator=g).to(torch.bfloat16)
    z = torch.randn(shape, generator=g).to(torch.bfloat16)
    wt = torch.randn(80 * 64, generator=g)
    assert 3 * y.numel() * 2 > 256 * 2**20
    say(f"norm streaming shape={shape} gate=True")
    yd, zd, wd = y.cuda(), z.cuda(), wt.cuda()
    out = ssd.gated_rmsnorm(yd, zd, wd, 1e-5, 1)
    ssd.gated_rmsnorm(yd, zd, wd, 1e-5, 1, out=yd)
    torch.cuda.synchronize()
    assert torch.equal(out, yd)
    e = MaxRelErr()
    wn = wt.numpy()
    for b in range(shape[0]):
        ref = oracle.gated_rmsnorm(_f64(y[b:b + 1]), _f64(z[b:b + 1]), wn, 1e-5, 1)
        e.add(_f64(out[b:b + 1]), ref)
    say(f"  err={e.value():.3e}")
    assert e.value() <= TOL["bf16"]
