"""Every workload at full size on the GPU, in the launch configuration the
benchmark times (ssd_forward with a preallocated workspace), against the fp64
oracle over the WHOLE output: max|dy| / max|y| and the same for the final
state, over every (batch, head, token, channel) of the configuration
("Transformers are SSMs", Knowl 1 gives the map; Knowl 2 its outputs Y and
h_final). The oracle runs one batch element at a time (rows are
independent), so host memory stays bounded; both storage types of the
inter-chunk states are checked against the same oracle run."""
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import TOL, MaxRelErr, oracle_batch, record_parity, say, to_dev

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny", "m125", "m2p7", "long16k", "nsweep16", "nsweep64", "nsweep128", "nsweep256"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_fullsize_whole_output(name):
    w = inputs.WORKLOADS[name]
    say(f"fullsize {name} {w.describe()}")
    inp = inputs.generate(w, seed=0)
    dev = to_dev(inp)
    storages = ["fp32", "bf16"] if w.dtype == "bf16" else ["fp32"]
    outs = {}
    for sd in storages:
        d = ssd.dims_of(dev["x"], dev["B"], w.chunk_size, sd)
        ws = ssd.alloc_workspace(d, "cuda")
        y = torch.empty_like(dev["x"])
        fin = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
        ssd.ssd_forward(d, dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], y, fin, ws, ws.numel())
        torch.cuda.synchronize()
        del ws
        assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
        outs[sd] = (y, fin)
    errs = {sd: (MaxRelErr(), MaxRelErr()) for sd in storages}
    for b in range(w.batch):
        y_ref, fin_ref = oracle_batch(inp, b)
        for sd in storages:
            y, fin = outs[sd]
            errs[sd][0].add(y[b].float().cpu().numpy(), y_ref[0])
            errs[sd][1].add(fin[b].cpu().numpy(), fin_ref[0])
    tol = TOL[w.dtype]
    for sd in storages:
        record_parity("forward", name, sd, errs[sd][0].value(), errs[sd][1].value(), tol)
    for sd in storages:
        assert errs[sd][0].value() <= tol and errs[sd][1].value() <= tol, sd


def test_streaming_copies_ragged_whole_output():
    """A forward whose data exceeds the 256 MiB last-level cache takes the
    non-temporal copies of x and the carried states; here with a ragged last
    chunk (77 of 256 tokens), so the partial-block copies take that policy
    too. Whole output against the oracle, both state storage types."""
    w = inputs.WORKLOADS["m2p7"].replace(name="stream_ragged", batch=3, seqlen=32 * 256 + 77)
    esz = 2
    bt = w.batch * w.seqlen
    footprint = (esz * bt * (2 * w.nheads * w.headdim + 2 * w.ngroups * w.dstate) + 8 * bt * w.nheads
                 + esz * w.batch * w.nchunks * w.nheads * w.headdim * w.dstate)
    assert footprint > 256 * 2**20
    say(f"fullsize streaming ragged {w.describe()} footprint {footprint / 2**20:.0f} MiB")
    inp = inputs.generate(w, seed=3)
    dev = to_dev(inp)
    outs = {}
    for sd in ("fp32", "bf16"):
        d = ssd.dims_of(dev["x"], dev["B"], w.chunk_size, sd)
        ws = ssd.alloc_workspace(d, "cuda")
        y = torch.empty_like(dev["x"])
        fin = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
        ssd.ssd_forward(d, dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], y, fin, ws, ws.numel())
        torch.cuda.synchronize()
        del ws
        assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
        outs[sd] = (y, fin)
    errs = {sd: (MaxRelErr(), MaxRelErr()) for sd in outs}
    for b in range(w.batch):
        y_ref, fin_ref = oracle_batch(inp, b)
        for sd, (y, fin) in outs.items():
            errs[sd][0].add(y[b].float().cpu().numpy(), y_ref[0])
            errs[sd][1].add(fin[b].cpu().numpy(), fin_ref[0])
    tol = TOL[w.dtype]
    for sd in outs:
        record_parity("forward", w.name, sd, errs[sd][0].value(), errs[sd][1].value(), tol)
    for sd in outs:
        assert errs[sd][0].value() <= tol and errs[sd][1].value() <= tol, sd


@pytest.mark.parametrize("name", ["m2p7", "long16k"])
def test_fullsize_gated_whole_output(name):
    """ssd_forward_gated (the output gate y * silu(z) in the chunk scan's
    epilogue, "Transformers are SSMs", Knowl 6) at full size with the states
    stored in bf16, as the benchmark times it, against the oracle's recurrence
    followed by the fp64 gate, over every output element; the final state is
    the ungated one."""
    import oracle

    w = inputs.WORKLOADS[name]
    say(f"fullsize gated {name} {w.describe()}")
    inp = inputs.generate(w, seed=0)
    z = inputs.generate_gate(w, seed=1)
    dev = to_dev(inp)
    y, fin = ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], w.chunk_size, "bf16",
                         z=z.to("cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    ey, ef = MaxRelErr(), MaxRelErr()
    for b in range(w.batch):
        y_ref, fin_ref = oracle_batch(inp, b)
        ey.add(y[b].float().cpu().numpy(), oracle.silu_gate(y_ref[0], z[b].float().numpy()))
        ef.add(fin[b].cpu().numpy(), fin_ref[0])
    tol = TOL[w.dtype]
    record_parity("gated", name, "bf16", ey.value(), ef.value(), tol)
    assert ey.value() <= tol and ef.value() <= tol
