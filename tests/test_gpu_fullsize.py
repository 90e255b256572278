"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (ssd_forward with a preallocated workspace), checked against the fp64
oracle on sampled (batch, head) pairs: the oracle runs the recurrence on just
those pairs, which is exact because pairs are independent."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import TOL, say, to_dev

pytestmark = pytest.mark.gpu

SAMPLES = 4


def sampled_pairs(w, seed):
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (w.batch - 1, w.nheads - 1)}
    while len(pairs) < min(SAMPLES, w.batch * w.nheads):
        pairs.add((int(rng.integers(w.batch)), int(rng.integers(w.nheads))))
    return sorted(pairs)


@pytest.mark.parametrize("name", ["m125", "m2p7", "long16k", "nsweep16", "nsweep64", "nsweep128",
                                  "nsweep256"])
@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_fullsize_sampled(name, state_dtype):
    w = inputs.WORKLOADS[name]
    say(f"fullsize {name} {w.describe()} state={state_dtype}")
    inp = inputs.generate(w, seed=0)
    dev = to_dev(inp)
    d = ssd.dims_of(dev["x"], dev["B"], w.chunk_size, state_dtype)
    ws = ssd.alloc_workspace(d, "cuda")
    y = torch.empty_like(dev["x"])
    fin = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
    ssd.ssd_forward(d, dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], y, fin, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    hpg = w.nheads // w.ngroups
    ys, yr, fs, fr = [], [], [], []
    for b, h in sampled_pairs(w, seed=len(name)):
        g = h // hpg
        sl = {
            "x": inp["x"][b:b + 1, :, h:h + 1], "dt": inp["dt"][b:b + 1, :, h:h + 1],
            "A": inp["A"][h:h + 1], "B": inp["B"][b:b + 1, :, g:g + 1],
            "C": inp["C"][b:b + 1, :, g:g + 1], "D": inp["D"][h:h + 1],
        }
        f = inputs.to_float64(sl)
        y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"])
        ys.append(y[b, :, h].float().cpu().numpy())
        yr.append(y_ref[0, :, 0])
        fs.append(fin[b, h].cpu().numpy())
        fr.append(fin_ref[0, 0])
    ey = oracle.rel_err(np.stack(ys), np.stack(yr))
    ef = oracle.rel_err(np.stack(fs), np.stack(fr))
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]
