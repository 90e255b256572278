"""The chunk scan's traffic probe (libssd_peak.so, ssd_peak_scan_traffic),
which bench.py times beside the kernel: its y must come out equal to x (every
x tile went through LDS to the right y rows), at shapes with several heads
per workgroup, groups, and chunk 0 (no carried state) and later chunks."""
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


@pytest.mark.parametrize("shape", SHAPES)
def test_scan_traffic_probe_copies_x_to_y(shape):
    path = os.path.join(os.path.dirname(ssd.LIB_PATH), "libssd_peak.so")
    if not os.path.exists(path):
        pytest.skip("libssd_peak.so not built")
    b, T, H, P, N, G, Q, hpw = shape
    nc = T // Q
    print(f"scan traffic probe {shape}", flush=True)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_peak_scan_traffic.argtypes = [vp] * 8 + [i64] * 8 + [vp]
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
                                   b, T, H, P, N, G, Q, hpw, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(y, x)
