"""C-ABI checks that need no GPU: the library loads, exports every function
include/ssd.h declares, and rejects bad arguments synchronously (before any
HIP call, so these run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

import mamba_ssd_scan_04_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULLP, SHAPE, UNSUP, MISAL, WS = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssd.so not built")
    return ssd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"ssd_forward", "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing",
            "ssd_chunk_scan", "ssd_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssd.h but not exported"


def test_version_and_strings(lib):
    assert ssd.ssd_abi_version() == 1
    for code in range(8):
        assert len(ssd.ssd_status_string(code)) > 0
    assert "unknown" in ssd.ssd_status_string(99)


def dims(**kw):
    base = dict(batch=2, seqlen=512, nheads=8, headdim=64, dstate=128, ngroups=2,
                chunk_size=256, dtype="bf16", state_dtype="fp32")
    base.update(kw)
    return ssd.make_dims(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, OK),
    (dict(batch=0), OK),
    (dict(seqlen=0), OK),
    (dict(seqlen=1000), OK),
    (dict(batch=-1), SHAPE),
    (dict(seqlen=-5), SHAPE),
    (dict(nheads=0), SHAPE),
    (dict(ngroups=3), SHAPE),
    (dict(chunk_size=0), SHAPE),
    (dict(headdim=48), UNSUP),
    (dict(headdim=256), UNSUP),
    (dict(dstate=8), UNSUP),
    (dict(dstate=512), UNSUP),
    (dict(chunk_size=16), OK),
    (dict(chunk_size=8), UNSUP),
    (dict(chunk_size=100), UNSUP),
    (dict(dtype=7), UNSUP),
    (dict(state_dtype=5), UNSUP),
    (dict(dtype="fp32", state_dtype="bf16"), UNSUP),
    (dict(dtype="bf16", state_dtype="bf16"), OK),
    (dict(dtype="fp32", headdim=16, dstate=16, chunk_size=64), OK),
    (dict(dtype="fp32", headdim=128, dstate=256, chunk_size=256), UNSUP),  # fp32 tile > LDS
    (dict(headdim=128, dstate=256, chunk_size=256), UNSUP),  # x + fp32 state tiles > LDS
    (dict(headdim=128, dstate=256, chunk_size=256, state_dtype="bf16"), OK),
    (dict(headdim=128, dstate=256, chunk_size=64), OK),      # 16 KB x + 128 KB fp32 state tile + vectors
    (dict(headdim=128, dstate=256, chunk_size=128), UNSUP),  # 32 KB x + 128 KB state tile
    (dict(headdim=128, dstate=256, chunk_size=64, state_dtype="bf16"), OK),
    (dict(headdim=64, dstate=256, chunk_size=256), OK),
])
def test_check_dims(lib, kw, code):
    assert ssd.ssd_check_dims(dims(**kw)) == code


def test_check_dims_null(lib):
    assert lib.ssd_check_dims(None) == NULLP
    assert lib.ssd_workspace_size(None) == 0


def test_workspace_size(lib):
    d = dims()
    nc = 2
    cs = 2 * 8 * nc * 256 * 4
    st = 2 * nc * 8 * 64 * 128 * 4
    assert ssd.ssd_workspace_size(d) == cs + st
    assert ssd.ssd_stage_sizes(d) == (cs, st)
    assert ssd.ssd_workspace_size(dims(state_dtype="bf16")) == cs + st // 2
    assert ssd.ssd_workspace_size(dims(headdim=48)) == 0
    assert ssd.ssd_workspace_size(dims(batch=0)) == 0
    # monotonic in every size
    w = ssd.ssd_workspace_size(d)
    for k, v in dict(batch=3, seqlen=513, nheads=10, headdim=128, dstate=256).items():
        bigger = dims(**{k: v, "state_dtype": "bf16"}) if k in ("headdim", "dstate") else dims(**{k: v})
        base = ssd.ssd_workspace_size(dims(state_dtype="bf16")) if k in ("headdim", "dstate") else w
        assert ssd.ssd_workspace_size(bigger) > base
    # ragged T rounds up to whole chunks
    assert ssd.ssd_workspace_size(dims(seqlen=300)) == ssd.ssd_workspace_size(dims(seqlen=512))


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_forward_argument_errors(lib):
    d = dims()
    ws = ssd.ssd_workspace_size(d)
    good = [_fake(0x100000 * (i + 1)) for i in range(10)]
    x, dt, A, B, C, D, y, fin, work = good[:9]
    f = lib.ssd_forward
    P = ctypes.byref
    assert f(P(d), None, dt, A, B, C, D, y, fin, work, ws, None) == NULLP
    assert f(P(d), x, dt, A, B, C, D, y, None, work, ws, None) == NULLP
    assert f(P(d), x, dt, A, B, C, D, y, fin, None, ws, None) == NULLP
    assert f(P(d), _fake(0x100008), dt, A, B, C, D, y, fin, work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, y, _fake(0x100004), work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, y, fin, work, ws - 1, None) == WS
    bad = dims(ngroups=3)
    assert f(P(bad), x, dt, A, B, C, D, y, fin, work, ws, None) == SHAPE
    # batch == 0 is a no-op that succeeds without touching any pointer
    assert f(P(dims(batch=0)), None, None, None, None, None, None, None, None, None, 0, None) == OK


def test_stage_argument_errors(lib):
    d = dims()
    P = ctypes.byref
    a = _fake(0x200000)
    assert lib.ssd_chunk_cumsum(P(d), None, a, a, None) == NULLP
    assert lib.ssd_chunk_cumsum(P(d), a, a, _fake(0x200002), None) == MISAL
    assert lib.ssd_chunk_state(P(d), a, a, a, a, None, None) == NULLP
    assert lib.ssd_chunk_cumsum_state(P(d), a, a, None, a, a, a, None) == NULLP
    assert lib.ssd_chunk_cumsum_state(P(d), a, a, a, a, _fake(0x200004), a, None) == MISAL
    assert lib.ssd_state_passing(P(d), a, a, None, None) == NULLP
    assert lib.ssd_chunk_scan(P(d), a, a, a, a, a, a, a, None, None) == NULLP
    assert lib.ssd_chunk_scan(P(dims(headdim=40)), a, a, a, a, a, a, a, a, None) == UNSUP
    # empty inputs: nothing to do, success without pointers
    e = dims(seqlen=0)
    assert lib.ssd_chunk_cumsum(P(e), None, None, None, None) == OK
    assert lib.ssd_chunk_state(P(e), None, None, None, None, None, None) == OK
    assert lib.ssd_chunk_cumsum_state(P(e), None, None, None, None, None, None, None) == OK
    assert lib.ssd_chunk_scan(P(e), None, None, None, None, None, None, None, None, None) == OK


def test_initial_state_argument_errors(lib):
    d = dims()
    ws = ssd.ssd_workspace_size(d)
    good = [_fake(0x100000 * (i + 1)) for i in range(11)]
    x, dt, A, B, C, D, ini, y, fin, work = good[:10]
    f = lib.ssd_forward_init
    P = ctypes.byref
    assert f(P(d), None, dt, A, B, C, D, ini, y, fin, work, ws, None) == NULLP
    assert f(P(d), x, dt, A, B, C, D, ini, y, None, work, ws, None) == NULLP
    assert f(P(d), x, dt, A, B, C, D, _fake(0x100004), y, fin, work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, ini, y, fin, work, ws - 1, None) == WS
    assert f(P(dims(ngroups=3)), x, dt, A, B, C, D, ini, y, fin, work, ws, None) == SHAPE
    assert f(P(dims(batch=0)), None, None, None, None, None, None, None, None, None, None, 0, None) == OK
    a = _fake(0x200000)
    assert lib.ssd_state_passing_init(P(d), a, a, a, None, None) == NULLP
    assert lib.ssd_state_passing_init(P(d), None, a, a, a, None) == NULLP
    assert lib.ssd_state_passing_init(P(d), a, a, _fake(0x200004), a, None) == MISAL
    assert lib.ssd_chunk_scan_init(P(d), a, a, a, a, a, a, a, None, None) == NULLP
    assert lib.ssd_chunk_scan_init(P(dims(headdim=40)), a, a, a, a, a, a, a, a, None) == UNSUP
    e = dims(seqlen=0)
    assert lib.ssd_chunk_scan_init(P(e), None, None, None, None, None, None, None, None, None) == OK


def test_gated_forward_argument_errors(lib):
    d = dims()
    ws = ssd.ssd_workspace_size(d)
    good = [_fake(0x400000 * (i + 1)) for i in range(11)]
    x, dt, A, B, C, D, z, y, fin, work = good[:10]
    f = lib.ssd_forward_gated
    P = ctypes.byref
    assert f(P(d), x, dt, A, B, C, D, None, None, y, fin, work, ws, None) == NULLP    # z required
    assert f(P(d), x, dt, A, B, C, D, None, _fake(0x400002), y, fin, work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, None, z, y, fin, work, ws - 1, None) == WS
    assert f(P(dims(batch=0)), None, None, None, None, None, None, None, None, None, None, None, 0, None) == OK


def test_step_argument_errors(lib):
    P = ctypes.byref
    a = _fake(0x300000)
    d = dims()
    assert lib.ssd_step(None, a, a, a, a, a, a, a, a, None) == NULLP
    assert lib.ssd_step(P(d), None, a, a, a, a, a, a, a, None) == NULLP
    assert lib.ssd_step(P(d), a, a, a, a, a, a, None, a, None) == NULLP
    assert lib.ssd_step(P(d), a, a, a, a, a, a, _fake(0x300008), a, None) == MISAL
    assert lib.ssd_step(P(dims(headdim=40)), a, a, a, a, a, a, a, a, None) == UNSUP
    assert lib.ssd_step(P(dims(ngroups=3)), a, a, a, a, a, a, a, a, None) == SHAPE
    # the sequence length and chunk size play no part in one step
    assert lib.ssd_step(P(dims(batch=0, seqlen=0, chunk_size=7)), None, None, None, None, None, None,
                        None, None, None) == OK


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ssd, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ssd, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        ssd.load_library()


def test_peak_probe_library_exports():
    """The attainable-peak probes the benchmark times (an MFMA loop and a
    streaming copy) are built beside the SSD library and reject bad
    arguments before launching anything."""
    path = os.path.join(os.path.dirname(ssd.LIB_PATH), "libssd_peak.so")
    if not os.path.exists(path):
        pytest.skip("libssd_peak.so not built")
    peak = ctypes.CDLL(path)
    peak.ssd_peak_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    peak.ssd_peak_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
    assert peak.ssd_peak_mfma_bf16(0, 10, _fake(0x1000), None) != 0
    assert peak.ssd_peak_mfma_bf16(4, 10, None, None) != 0
    assert peak.ssd_peak_stream(_fake(0x1000), _fake(0x2000), 0, 4, None) != 0
    assert peak.ssd_peak_stream(_fake(0x1008), _fake(0x2000), 16, 4, None) != 0
    peak.ssd_peak_stream_pieces.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert peak.ssd_peak_stream_pieces(_fake(0x1000), _fake(0x2000), 0, None) != 0
    assert peak.ssd_peak_stream_pieces(_fake(0x1000), _fake(0x2008), 16, None) != 0
    assert peak.ssd_peak_stream_pieces(None, _fake(0x2000), 16, None) != 0
    # the chunk scan's traffic probe: a null pointer, then shapes it does not
    # cover (T not a multiple of Q, Q above 256, P not a multiple of 8, a tile
    # that is not whole 64-lane groups), all rejected before any launch
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    peak.ssd_peak_scan_traffic.argtypes = [vp] * 8 + [i64] * 9 + [vp]
    ptrs = [_fake(0x10000 * (i + 1)) for i in range(8)]
    assert peak.ssd_peak_scan_traffic(None, *ptrs[1:], 1, 512, 2, 64, 128, 1, 256, 1, 0, None) != 0
    assert peak.ssd_peak_scan_traffic(*ptrs, 1, 500, 2, 64, 128, 1, 256, 1, 0, None) == -1
    assert peak.ssd_peak_scan_traffic(*ptrs, 1, 1024, 2, 64, 128, 1, 512, 1, 0, None) == -1
    assert peak.ssd_peak_scan_traffic(*ptrs, 1, 512, 2, 60, 128, 1, 256, 1, 0, None) == -1
    assert peak.ssd_peak_scan_traffic(*ptrs, 1, 512, 2, 16, 16, 1, 32, 1, 0, None) == -1
    # the chunk state's traffic probe: a null pointer, then shapes it does not
    # cover (T not a multiple of Q, Q not a multiple of 32, P or N not a
    # multiple of 64, 3 heads per workgroup)
    peak.ssd_peak_state_traffic.argtypes = [vp] * 5 + [i64] * 9 + [vp]
    assert peak.ssd_peak_state_traffic(None, *ptrs[1:5], 1, 512, 4, 64, 128, 1, 256, 4, 0, None) != 0
    assert peak.ssd_peak_state_traffic(*ptrs[:5], 1, 500, 4, 64, 128, 1, 256, 4, 0, None) == -1
    assert peak.ssd_peak_state_traffic(*ptrs[:5], 1, 512, 4, 64, 128, 1, 16, 4, 0, None) == -1
    assert peak.ssd_peak_state_traffic(*ptrs[:5], 1, 512, 4, 32, 128, 1, 256, 4, 0, None) == -1
    assert peak.ssd_peak_state_traffic(*ptrs[:5], 1, 512, 4, 64, 16, 1, 256, 4, 0, None) == -1
    assert peak.ssd_peak_state_traffic(*ptrs[:5], 1, 512, 6, 64, 128, 1, 256, 3, 0, None) == -1


def test_varlen_forward_argument_errors(lib):
    d = dims()
    ws = ssd.ssd_workspace_size(d)
    good = [_fake(0x500000 * (i + 1)) for i in range(11)]
    x, dt, A, B, C, D, seq, y, fin, work = good[:10]
    f = lib.ssd_forward_varlen
    P = ctypes.byref
    assert f(P(d), x, dt, A, B, C, D, None, None, y, fin, work, ws, None) == NULLP    # seq_idx required
    assert f(P(d), x, dt, A, B, C, D, None, _fake(0x500002), y, fin, work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, None, seq, y, fin, work, ws - 1, None) == WS
    assert f(P(d), None, dt, A, B, C, D, None, seq, y, fin, work, ws, None) == NULLP
    assert f(P(dims(ngroups=3)), x, dt, A, B, C, D, None, seq, y, fin, work, ws, None) == SHAPE
    # every shape the plain forward accepts leaves room for the chunk's ids in LDS
    big = dims(headdim=128, dstate=256, chunk_size=64)
    assert f(P(big), x, dt, A, B, C, D, None, seq, y, fin, work, ssd.ssd_workspace_size(big) - 1, None) == WS
    assert f(P(dims(batch=0)), None, None, None, None, None, None, None, None, None, None, None, 0, None) == OK


def test_varlen_gated_forward_argument_errors(lib):
    d = dims()
    ws = ssd.ssd_workspace_size(d)
    good = [_fake(0x700000 * (i + 1)) for i in range(11)]
    x, dt, A, B, C, D, seq, z, y, fin, work = good
    f = lib.ssd_forward_varlen_gated
    P = ctypes.byref
    assert f(P(d), x, dt, A, B, C, D, None, seq, None, y, fin, work, ws, None) == NULLP     # z required
    assert f(P(d), x, dt, A, B, C, D, None, None, z, y, fin, work, ws, None) == NULLP     # seq_idx required
    assert f(P(d), x, dt, A, B, C, D, None, _fake(0x700002), z, y, fin, work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, None, seq, _fake(0x700008), y, fin, work, ws, None) == MISAL
    assert f(P(d), x, dt, A, B, C, D, None, seq, z, y, fin, work, ws - 1, None) == WS
    assert f(P(dims(ngroups=3)), x, dt, A, B, C, D, None, seq, z, y, fin, work, ws, None) == SHAPE
    assert f(P(dims(batch=0)), *([None] * 12), 0, None) == OK


def test_shard_entry_points_argument_errors(lib):
    P = ctypes.byref
    a = _fake(0x600000)
    d = dims()
    assert lib.ssd_total_decay(None, a, a, a, None) == NULLP
    assert lib.ssd_total_decay(P(d), None, a, a, None) == NULLP
    assert lib.ssd_total_decay(P(d), a, a, _fake(0x600004), None) == MISAL
    assert lib.ssd_total_decay(P(dims(headdim=40)), a, a, a, None) == UNSUP
    assert lib.ssd_total_decay(P(dims(batch=0)), None, None, None, None) == OK
    assert lib.ssd_fold_states(P(d), -1, a, a, None, a, None) == SHAPE
    assert lib.ssd_fold_states(P(d), 4, None, a, None, a, None) == NULLP
    assert lib.ssd_fold_states(P(d), 4, a, a, None, None, None) == NULLP
    assert lib.ssd_fold_states(P(d), 4, a, a, _fake(0x600008), a, None) == MISAL
    assert lib.ssd_fold_states(P(dims(nheads=0)), 4, a, a, None, a, None) == SHAPE
    assert lib.ssd_fold_states(P(dims(batch=0)), 4, None, None, None, None, None) == OK


def test_gated_rmsnorm_argument_errors(lib):
    P = ctypes.byref
    a = _fake(0x700000)
    d = dims()
    f = lib.ssd_gated_rmsnorm
    assert f(None, a, None, a, ctypes.c_float(1e-5), 1, a, None) == NULLP
    assert f(P(d), None, None, a, ctypes.c_float(1e-5), 1, a, None) == NULLP
    assert f(P(d), a, None, None, ctypes.c_float(1e-5), 1, a, None) == NULLP
    assert f(P(d), a, None, a, ctypes.c_float(1e-5), 0, a, None) == SHAPE
    assert f(P(d), a, None, a, ctypes.c_float(1e-5), 3, a, None) == SHAPE         # 3 does not divide 8 * 64
    assert f(P(d), a, None, a, ctypes.c_float(1e-5), 128, a, None) == UNSUP       # 4 channels per group
    assert f(P(d), a, _fake(0x700004), a, ctypes.c_float(1e-5), 1, a, None) == MISAL
    assert f(P(dims(dtype=7)), a, None, a, ctypes.c_float(1e-5), 1, a, None) == UNSUP
    assert f(P(dims(seqlen=0)), None, None, None, ctypes.c_float(1e-5), 1, None, None) == OK


# ---- the binding's argument checks (CPU tensors: rejected before any call) ----

def _inputs(dtype=None, **over):
    import torch
    xt = dtype or torch.bfloat16
    b, T, H, P, N, G = 2, 64, 4, 16, 16, 2
    t = {"x": torch.zeros(b, T, H, P, dtype=xt), "dt": torch.zeros(b, T, H), "A": torch.zeros(H),
         "B": torch.zeros(b, T, G, N, dtype=xt), "C": torch.zeros(b, T, G, N, dtype=xt), "D": torch.zeros(H)}
    t.update(over)
    return t


@pytest.mark.parametrize("over,exc,what", [
    (dict(dt="bf16"), TypeError, "dt must be torch.float32"),
    (dict(A="short"), ValueError, "A must have shape"),
    (dict(D="f64"), TypeError, "D must be torch.float32"),
    (dict(C="f32"), TypeError, "C must be torch.bfloat16"),
    (dict(C="short"), ValueError, "C must have shape"),
    (dict(dt="short"), ValueError, "dt must have shape"),
    (dict(), ValueError, "must be on a CUDA device"),
])
def test_binding_rejects_bad_tensors(lib, over, exc, what):
    import torch
    t = _inputs()
    for k, v in over.items():
        if v == "bf16":
            t[k] = t[k].to(torch.bfloat16)
        elif v == "f32":
            t[k] = t[k].float()
        elif v == "f64":
            t[k] = t[k].double()
        elif v == "short":
            t[k] = t[k][..., :-1].contiguous() if t[k].dim() > 1 else t[k][:-1].contiguous()
    with pytest.raises(exc, match=what):
        ssd.forward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 32)


def test_binding_rejects_bad_b_and_optional_tensors(lib):
    import torch
    t = _inputs()
    with pytest.raises(TypeError, match="B must have x's type"):
        ssd.forward(t["x"], t["dt"], t["A"], t["B"].float(), t["C"], t["D"], 32)
    with pytest.raises(ValueError, match="B must be"):
        ssd.forward(t["x"], t["dt"], t["A"], t["B"][:1].contiguous(), t["C"], t["D"], 32)
    with pytest.raises(ValueError, match="initial_state must have shape"):
        ssd.forward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 32,
                    initial_state=torch.zeros(2, 4, 16, 15))
    with pytest.raises(TypeError, match="seq_idx must be torch.int32"):
        ssd.forward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 32,
                    seq_idx=torch.zeros(2, 64, dtype=torch.int64))
    with pytest.raises(TypeError, match="z must be torch.bfloat16"):
        ssd.forward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 32, z=torch.zeros(2, 64, 4, 16))
    d = ssd.dims_of(t["x"], t["B"], 32, "fp32")
    with pytest.raises(TypeError, match="states must be torch.float32"):
        ssd.ssd_state_passing(d, torch.zeros(2, 4, 2, 32), torch.zeros(2, 2, 4, 16, 16, dtype=torch.bfloat16),
                              torch.zeros(2, 4, 16, 16))
    with pytest.raises(ValueError, match="cs must have shape"):
        ssd.ssd_chunk_cumsum(d, t["dt"], t["A"], torch.zeros(2, 4, 2, 31))
    with pytest.raises(ValueError, match="state must have shape"):
        ssd.step(t["x"][:, 0].contiguous(), t["dt"][:, 0].contiguous(), t["A"], t["B"][:, 0].contiguous(),
                 t["C"][:, 0].contiguous(), t["D"], torch.zeros(2, 4, 16, 17))
    with pytest.raises(ValueError, match="weight must be"):
        ssd.gated_rmsnorm(t["x"], None, torch.zeros(3))


def test_check_dims_rejects_chunk_spans_past_31_bits(lib):
    # one chunk's rows of x span Q*H*P*esize bytes, addressed with 32-bit offsets
    assert ssd.ssd_check_dims(dims(nheads=32767, ngroups=1, headdim=128, dstate=128)) == OK
    assert ssd.ssd_check_dims(dims(nheads=32768, ngroups=1, headdim=128, dstate=128)) == UNSUP
    assert ssd.ssd_check_dims(dims(dtype="fp32", nheads=32767, ngroups=1, headdim=128, dstate=64,
                                   chunk_size=128)) == OK
    assert ssd.ssd_check_dims(dims(dtype="fp32", nheads=32768, ngroups=1, headdim=128, dstate=64,
                                   chunk_size=128)) == UNSUP
    # B and C rows: Q*G*N*esize
    assert ssd.ssd_check_dims(dims(dtype="fp32", nheads=8192, ngroups=8192, headdim=16, dstate=256,
                                   chunk_size=256)) == UNSUP
    assert ssd.ssd_check_dims(dims(dtype="fp32", nheads=8191, ngroups=8191, headdim=16, dstate=256,
                                   chunk_size=256)) == OK


def test_noalloc_forward_argument_errors(lib):
    """The allocation-free forward checks its arguments and its size limit
    before any HIP call: dims, the fixed scratch's size, then pointers."""
    P = ctypes.byref
    a = _fake(0x400000)
    f = lib.ssd_forward_noalloc
    assert ssd.ssd_noalloc_scratch_bytes() == 64 << 20
    assert "fixed device scratch" in ssd.ssd_status_string(7)
    d = dims()   # 2 x 512 tokens, 8 heads of 64 x 128: well under 64 MiB of workspace
    assert ssd.ssd_workspace_size(d) <= ssd.ssd_noalloc_scratch_bytes()
    assert f(P(d), None, a, a, a, a, a, a, a, None) == NULLP
    assert f(P(d), a, a, a, a, a, a, a, None, None) == NULLP
    assert f(P(dims(ngroups=3)), a, a, a, a, a, a, a, a, None) == SHAPE
    assert f(P(dims(headdim=48)), a, a, a, a, a, a, a, a, None) == UNSUP
    big = dims(batch=8, seqlen=4096, nheads=80)   # the 2.7B-layer shape: ~346 MB of fp32 states
    assert ssd.ssd_workspace_size(big) > ssd.ssd_noalloc_scratch_bytes()
    assert f(P(big), a, a, a, a, a, a, a, a, None) == 7
    assert f(P(dims(batch=0)), None, None, None, None, None, None, None, None, None) == OK


def test_prepared_records_one_checked_call(lib):
    """ssd.prepared runs a wrapper's checks once and records its C call
    without making it; a function that makes no C call is refused."""
    import torch
    d = dims()
    a = 0x500000
    call = ssd.prepared(ssd.ssd_forward, d, a, a, a, a, a, a, a, a, a, 1 << 30, stream=0)
    assert callable(call)
    with pytest.raises(ValueError, match="made 0 C calls"):
        ssd.prepared(lambda: None)
    t = _inputs()
    with pytest.raises(ValueError, match="must be on a CUDA device"):   # the checks still run
        ssd.prepared(ssd.ssd_forward, ssd.dims_of(t["x"], t["B"], 32), t["x"], t["dt"], t["A"], t["B"], t["C"],
                     t["D"], torch.empty_like(t["x"]), torch.zeros(2, 4, 16, 16), a, 1 << 30, stream=0)
