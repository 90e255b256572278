"""The allocation-free forward (ssd_forward_noalloc) through the C ABI against
ssd_forward on the same inputs: bitwise equal outputs, on two calls in a row
(the second with a smaller input, so that the fixed scratch holds the first
call's data when the second starts), and once more after a larger call of
ssd_forward. Runs alone or after the other tests."""
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import say, to_dev, workload

pytestmark = pytest.mark.gpu


def run_both(w, seed, state_dtype):
    g = to_dev(inputs.generate(w, seed=seed))
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, state_dtype)
    assert ssd.ssd_workspace_size(d) <= ssd.ssd_noalloc_scratch_bytes()
    fin_shape = (w.batch, w.nheads, w.dstate, w.headdim)
    y0 = torch.full_like(g["x"], float("nan"))
    f0 = torch.full(fin_shape, float("nan"), device="cuda")
    ws = ssd.alloc_workspace(d, "cuda")
    ssd.ssd_forward(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y0, f0, ws, ws.numel())
    y1 = torch.full_like(g["x"], float("nan"))
    f1 = torch.full(fin_shape, float("nan"), device="cuda")
    ssd.ssd_forward_noalloc(d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y1, f1)
    torch.cuda.synchronize()
    return y0, f0, y1, f1


@pytest.mark.parametrize("state_dtype", ["bf16", "fp32"])
def test_noalloc_matches_forward_on_two_calls(state_dtype):
    first = workload("m125", batch=2, seqlen=2048, nheads=12)
    second = workload("m125", batch=1, seqlen=700, nheads=4)    # smaller: reuses stale scratch
    for w, seed in ((first, 51), (second, 52)):
        say(f"noalloc case {w.describe()} state={state_dtype}")
        y0, f0, y1, f1 = run_both(w, seed, state_dtype)
        assert torch.isfinite(y1.float()).all() and torch.isfinite(f1).all()
        assert torch.equal(y0, y1) and torch.equal(f0, f1)


def test_noalloc_fp32_inputs_and_rejection():
    w = workload("tiny")
    y0, f0, y1, f1 = run_both(w, 53, "fp32")
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    big = workload("m2p7")
    d = ssd.make_dims(big.batch, big.seqlen, big.nheads, big.headdim, big.dstate, big.ngroups, big.chunk_size,
                      "bf16", "bf16")
    x = torch.empty((1,), device="cuda")
    with pytest.raises(ssd.SsdError, match="fixed device scratch"):
        ssd.ssd_forward_noalloc(d, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                x.data_ptr(), x.data_ptr(), x.data_ptr(), stream=torch.cuda.current_stream().cuda_stream)
