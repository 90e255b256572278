"""The traffic probes (libssd_peak.so) that bench.py times beside the
kernels. The chunk scan's (ssd_peak_scan_traffic): its y must come out equal
to x (every x tile went through LDS to the right y rows), at shapes with
several heads per workgroup, groups, and chunk 0 (no carried state) and later
chunks. The chunk state's (ssd_peak_state_traffic): cs must equal dt and each
state the head's last 32 x rows of the chunk, repeated (every copy went
through the LDS ring to the right place)."""
import ctypes
import os

import pytest
import torch

import mamba_ssd_scan_04_amd as ssd

pytestmark = pytest.mark.gpu

SHAPES = [  # b, T, H, P, N, G, Q, heads per workgroup
    (2, 512, 6, 64, 128, 2, 256, 2),
    (1, 256, 3, 32, 64, 1, 128, 3),
    (2, 1024, 8, 64, 64, 1, 256, 4),
]


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_scan_traffic_probe_copies_x_to_y(shape, nt):
    path = os.path.join(os.path.dirname(ssd.LIB_PATH), "libssd_peak.so")
    if not os.path.exists(path):
        pytest.skip("libssd_peak.so not built")
    b, T, H, P, N, G, Q, hpw = shape
    nc = T // Q
    print(f"scan traffic probe {shape} nt={nt}", flush=True)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_peak_scan_traffic.argtypes = [vp] * 8 + [i64] * 9 + [vp]
    g = torch.Generator(device="cpu").manual_seed(7)
    dev = torch.device("cuda:0")
    x = torch.randn(b, T, H, P, generator=g).to(torch.bfloat16).to(dev)
    Bm = torch.randn(b, T, G, N, generator=g).to(torch.bfloat16).to(dev)
    Cm = torch.randn(b, T, G, N, generator=g).to(torch.bfloat16).to(dev)
    st = torch.randn(b, nc, H, P, N, generator=g).to(torch.bfloat16).to(dev)
    dt = torch.rand(b, T, H, generator=g).to(dev)
    cs = torch.randn(b, H, nc, Q, generator=g).to(dev)
    y = torch.zeros_like(x)
    nhb = -(-(H // G) // hpw)
    sink = torch.zeros(b * nc * G * nhb, device=dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.ssd_peak_scan_traffic(ptr(x), ptr(Bm), ptr(Cm), ptr(st), ptr(dt), ptr(cs), ptr(y), ptr(sink),
                                   b, T, H, P, N, G, Q, hpw, nt,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(y, x)


STATE_SHAPES = [  # b, T, H, P, N, G, Q, heads per workgroup
    (2, 512, 8, 64, 128, 1, 256, 4),
    (1, 768, 6, 64, 64, 2, 128, 2),
    (2, 256, 3, 64, 256, 3, 64, 1),
    (1, 512, 4, 128, 128, 1, 32, 2),
]


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("shape", STATE_SHAPES)
def test_state_traffic_probe_copies(shape, nt):
    path = os.path.join(os.path.dirname(ssd.LIB_PATH), "libssd_peak.so")
    if not os.path.exists(path):
        pytest.skip("libssd_peak.so not built")
    b, T, H, P, N, G, Q, hpw = shape
    nc = T // Q
    print(f"state traffic probe {shape} nt={nt}", flush=True)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_peak_state_traffic.argtypes = [vp] * 5 + [i64] * 9 + [vp]
    g = torch.Generator(device="cpu").manual_seed(11)
    dev = torch.device("cuda:0")
    x = torch.randn(b, T, H, P, generator=g).to(torch.bfloat16).to(dev)
    Bm = torch.randn(b, T, G, N, generator=g).to(torch.bfloat16).to(dev)
    dt = torch.rand(b, T, H, generator=g).to(dev)
    cs = torch.zeros(b, H, nc, Q, device=dev)
    st = torch.zeros(b, nc, H, P, N, dtype=torch.bfloat16, device=dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.ssd_peak_state_traffic(ptr(x), ptr(Bm), ptr(dt), ptr(cs), ptr(st), b, T, H, P, N, G, Q, hpw, nt,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(cs, dt.view(b, nc, Q, H).permute(0, 3, 1, 2))
    last = x.view(b, nc, Q, H, P)[:, :, -32:].permute(0, 1, 3, 2, 4)
    want = last.unsqueeze(3).expand(-1, -1, -1, N // 32, -1, -1)
    assert torch.equal(st.view(want.shape), want)


@pytest.mark.parametrize("nvec", [1, 255, 256, 257, 4096 * 3 + 5])
def test_stream_probes_copy_exactly(nvec):
    """Both streaming copies of the attainable-peak figure (grid-stride, and
    one 4 KB piece per workgroup) copy exactly n 16-byte vectors: every
    vector, including a ragged last piece, and nothing past the end."""
    path = os.path.join(os.path.dirname(ssd.LIB_PATH), "libssd_peak.so")
    if not os.path.exists(path):
        pytest.skip("libssd_peak.so not built")
    print(f"stream probes nvec={nvec}", flush=True)
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.ssd_peak_stream.argtypes = [vp, vp, i64, i64, vp]
    lib.ssd_peak_stream_pieces.argtypes = [vp, vp, i64, vp]
    dev = torch.device("cuda:0")
    src = torch.arange(nvec * 4 + 4, dtype=torch.int32, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for call in (lambda d: lib.ssd_peak_stream(src.data_ptr(), d.data_ptr(), nvec, 4, s),
                 lambda d: lib.ssd_peak_stream_pieces(src.data_ptr(), d.data_ptr(), nvec, s)):
        dst = torch.full_like(src, -1)
        assert call(dst) == 0
        torch.cuda.synchronize()
        assert torch.equal(dst[:nvec * 4], src[:nvec * 4])
        assert torch.equal(dst[nvec * 4:], torch.full((4,), -1, dtype=torch.int32, device=dev))
