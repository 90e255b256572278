"""The benchmark's byte and flop accounting (CPU): the per-token method bytes
and the three-kernel design bytes at the 2.7B-layer shape against the figures
derived by hand from the layouts, and the algorithmic work of each kernel
against its definition at a small shape."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mamba_ssd_scan_04_amd import inputs  # noqa: E402


def test_method_bytes_per_token_at_the_layer_shape():
    """x, B, C in and y out in bf16 (2 bytes), dt in fp32, plus the final state:
    2*(2*80*64 + 2*128) + 4*80 = 21,328 bytes per token, and 8*80*128*64*4
    bytes of final state over the batch."""
    w = inputs.WORKLOADS["m2p7"]
    tokens = w.batch * w.seqlen
    assert bench.method_bytes(w) == tokens * (2 * (2 * 80 * 64 + 2 * 128) + 4 * 80) + 8 * 80 * 128 * 64 * 4


def test_design_bytes_at_the_layer_shape():
    """The three launches with bf16 states: chunk state reads x, B, dt and
    writes cs and S; state passing reads S and writes h_in and the final
    state (plus the chunk totals); chunk scan reads x, B, C, dt, cs and
    h_in (no h_0) and writes y."""
    w = inputs.WORKLOADS["m2p7"]
    b, T, H, P, N, G, Q, nc = 8, 4096, 80, 64, 128, 1, 256, 16
    st = b * nc * H * N * P * 2
    work = bench.kernel_work(w, 2)
    assert work["ssd_chunk_state"]["bytes"] == 2 * b * T * (H * P + G * N) + 4 * b * T * H + 4 * b * H * nc * Q + st
    assert work["ssd_state_passing"]["bytes"] == 2 * st + 4 * b * H * N * P + 4 * b * H * nc
    assert work["ssd_chunk_scan"]["bytes"] == (2 * b * T * (2 * H * P + 2 * G * N) + 8 * b * T * H
                                               + b * (nc - 1) * H * N * P * 2)
    total = sum(work[k]["bytes"] for k in bench.KERNELS)
    assert abs(total - 1.755e9) < 0.001e9


def test_flops_match_the_definitions():
    """Chunk state: 2 N P flops per token and head; chunk scan: the causal
    triangle (with diagonal) of C B^T once per group and of the masked product
    per head, plus 2 N P per token and head for the carried state outside the
    first chunk."""
    w = inputs.WORKLOADS["m2p7"].replace(batch=1, seqlen=512, nheads=4, ngroups=2, dstate=32, headdim=16,
                                         chunk_size=128)
    work = bench.kernel_work(w, 4)
    b, T, H, P, N, G, Q = 1, 512, 4, 16, 32, 2, 128
    nc = T // Q
    assert work["ssd_chunk_state"]["flops"] == 2 * b * T * H * N * P + b * T * H
    tri = Q * (Q + 1)
    assert work["ssd_chunk_scan"]["flops"] == b * nc * (G * N * tri + H * P * tri) + 2 * b * (T - Q) * H * N * P


def test_traffic_records_match_the_kernel_sources():
    """The committed rocprofv3 traffic records (profiles/pmc_*.json) were taken
    on the current kernel sources, so the benchmark reports the dominant
    kernel's measured HBM bytes (roofline.traffic) instead of null; and each
    record's bytes stay within 2% of the kernel's algorithmic bytes."""
    for kern in bench.KERNELS:
        for sd in ("bf16", "fp32"):
            got = bench.measured_traffic(kern, "m2p7", sd)
            assert got is not None, f"{kern} {sd}: no record for the current source"
            alg = bench.kernel_work(inputs.WORKLOADS["m2p7"], 2 if sd == "bf16" else 4)[kern]["bytes"]
            assert abs(got / alg - 1.0) < 0.02, (kern, sd, got, alg)
