"""GPU parity for the sequence-parallel path of Knowl 8 run on one device:
shards from a zero state, their total log-decays (ssd_total_decay), the
shard chain (ssd_fold_states) and the shards again from their entering
states (ssd_forward_init), against the fp64 oracle on the whole sequence."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_04_amd as ssd
import oracle
from mamba_ssd_scan_04_amd import inputs
from gpu_helpers import MaxRelErr, oracle_batch, record_parity, TOL, say, to_dev, workload

pytestmark = pytest.mark.gpu


def check(w, inp, bounds, state_dtype="fp32", init=None):
    say(f"case {w.describe()} shards={bounds} state={state_dtype} init={init is not None}")
    d = to_dev(inp)
    y, fin = ssd.forward_sharded(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_size, bounds,
                                 state_dtype, None if init is None else init.to("cuda"))
    torch.cuda.synchronize()
    f = inputs.to_float64(inp)
    y_ref, fin_ref = oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"],
                                       init=None if init is None else init.numpy().astype(np.float64))
    ey = oracle.rel_err(y.float().cpu().numpy().astype(np.float64), y_ref)
    ef = oracle.rel_err(fin.cpu().numpy().astype(np.float64), fin_ref)
    say(f"  err_y={ey:.3e} err_final={ef:.3e}")
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype], (ey, ef)


def test_tiny_fp32_shards():
    w = workload("tiny", batch=2, seqlen=256)
    check(w, inputs.generate_slow_decay(w, seed=50), [0, 64, 100, 256])


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("with_init", [False, True])
def test_m125_shape_shards(state_dtype, with_init):
    w = workload("m125", batch=2, seqlen=1000, nheads=4)
    init = inputs.generate_initial_state(w, seed=51) if with_init else None
    check(w, inputs.generate_slow_decay(w, seed=51), [0, 250, 500, 751, 1000], state_dtype, init)


def test_one_shard_is_the_forward():
    w = workload("m125", batch=1, seqlen=300, nheads=3)
    check(w, inputs.generate_slow_decay(w, seed=52), [0, 300])


def test_total_decay_is_the_sum():
    """Lambda[b,h] = A_h sum_t dt[b,t,h], against the fp64 sum of the same bits."""
    w = workload("m125", batch=3, seqlen=777, nheads=70)
    inp = inputs.generate(w, seed=53)
    d = ssd.dims_of(inp["x"], inp["B"], w.chunk_size, "fp32")
    tot = torch.empty((3, 70), dtype=torch.float32, device="cuda")
    ssd.ssd_total_decay(d, inp["dt"].cuda(), inp["A"].cuda(), tot)
    torch.cuda.synchronize()
    ref = inputs.to_float64(inp)["dt"].sum(axis=1) * inputs.to_float64(inp)["A"][None, :]
    assert np.max(np.abs(tot.cpu().numpy() - ref) / np.abs(ref)) < 1e-5


@pytest.mark.parametrize("name", ["long16k"])
def test_fullsize_eight_shards_whole_output(name):
    """The long-context workload cut into 8 shards of 2048 tokens (each shard
    at the shape one of 8 GPUs would run), against the oracle on the whole
    sequence over the whole output."""
    w = inputs.WORKLOADS[name]
    say(f"fullsize shards {name} {w.describe()}")
    inp = inputs.generate(w, seed=0)
    d = to_dev(inp)
    bounds = [k * w.seqlen // 8 for k in range(9)]
    y, fin = ssd.forward_sharded(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_size, bounds)
    torch.cuda.synchronize()
    ey, ef = MaxRelErr(), MaxRelErr()
    for b in range(w.batch):
        y_ref, fin_ref = oracle_batch(inp, b)
        ey.add(y[b].float().cpu().numpy(), y_ref[0])
        ef.add(fin[b].cpu().numpy(), fin_ref[0])
    record_parity("shards8", name, "bf16", ey.value(), ef.value(), TOL[w.dtype])
    assert ey.value() <= TOL[w.dtype] and ef.value() <= TOL[w.dtype]


def test_fold_chain_against_fp64():
    """ssd_fold_states alone: H_0 = init (or 0), H_{k+1} = exp(L_k) H_k + F_k,
    against the same chain in fp64 on the same bits, for K = 0, 1 and 5."""
    g = torch.Generator().manual_seed(54)
    b, H, N, P = 2, 3, 16, 32
    d = ssd.make_dims(b, 64, H, P, N, 1, 32, "fp32", "fp32")
    for K in (0, 1, 5):
        for with_init in (False, True):
            tot = -torch.rand((K, b, H), generator=g) * 3.0
            fin = torch.randn((K, b, H, N, P), generator=g)
            ini = torch.randn((b, H, N, P), generator=g) if with_init else None
            ent = torch.full((K + 1, b, H, N, P), float("nan"), device="cuda")
            ssd.ssd_fold_states(d, K, tot.cuda() if K else None, fin.cuda() if K else None,
                                None if ini is None else ini.cuda(), ent)
            torch.cuda.synchronize()
            ref = np.zeros((K + 1, b, H, N, P))
            run = np.zeros((b, H, N, P)) if ini is None else ini.numpy().astype(np.float64)
            for k in range(K):
                ref[k] = run
                run = np.exp(tot[k].numpy().astype(np.float64))[:, :, None, None] * run + fin[k].numpy()
            ref[K] = run
            got = ent.cpu().numpy().astype(np.float64)
            assert np.all(np.isfinite(got))
            assert oracle.rel_err(got, ref) < 1e-5, (K, with_init)
