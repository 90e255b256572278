"""Benchmark: SSD chunked forward tokens/s on one MI355X, with roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload m2p7]
                    [--state-dtype fp32|bf16] [--no-cpu-baseline]

One step is one ssd_forward call (three launches: the chunk-state kernel
with the in-chunk prefix sums formed inside it, state passing, chunk scan)
over one batch of seeded synthetic input already resident in HBM; its wall
clock gives tokens/s. Each kernel's average duration is measured in a second
timed loop that makes the same launches through the stage entry points with
HIP events between them on the launch stream. Rank 0 prints one JSON line.

Beside the headline figures the line carries: per-call medians of the
forward with warm caches and with a 512 MB scrub written between calls (cold
last-level cache); the path's bytes against the HBM peak, both the method's
compulsory bytes and the four-kernel design's; the attainable peaks of a bare
MFMA loop and a bare streaming copy on this chip; the other storage type of
the inter-chunk states; the gated forward, alone and followed by the
RMSNorm in place; the forward over rows packing
several documents; one GPU's share of an 8-way context-parallel forward; and
the decoding step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/sec at 2.7B-layer shape (L=4096, N=128); % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16, TFLOP/s
MFMA_F32_PEAK_TFS = 157.3
# the launches of ssd_forward: ssd_chunk_cumsum_state runs the chunk-state
# kernel with the in-chunk prefix sums formed inside it
KERNELS = ["ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan"]
SOURCES = {"ssd_chunk_cumsum": "chunk_cumsum.hip", "ssd_chunk_state": "chunk_state.hip",
           "ssd_state_passing": "state_passing.hip", "ssd_chunk_scan": "chunk_scan_impl.hpp"}


def kernel_work(w, state_bytes: int) -> dict:
    """Algorithmic bytes and flops per launch of each kernel (the bytes each
    must move at minimum given its inputs and outputs, and the flops of the
    method's contractions: causal lower triangle incl. the diagonal, C B^T
    once per group)."""
    b, T, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    nc = w.nchunks
    e = 2 if w.dtype == "bf16" else 4
    st = b * nc * H * N * P * state_bytes           # one pass over the chunk states
    st_in = b * (nc - 1) * H * N * P * state_bytes  # carried states read (h_0 = 0 is known)
    Qc = T / nc                                      # mean chunk length
    return {
        "ssd_chunk_cumsum": {"bytes": 4 * b * T * H + 4 * b * H * nc * Q, "flops": b * T * H},
        # with the prefix sums formed inside: reads x, B, dt; writes cs and the states
        "ssd_chunk_state": {"bytes": e * b * T * (H * P + G * N) + 4 * b * T * H + 4 * b * H * nc * Q + st,
                            "flops": 2 * b * T * H * N * P + b * T * H},
        "ssd_state_passing": {"bytes": 2 * st + 4 * b * H * N * P + 4 * b * H * nc,
                              "flops": 2 * b * nc * H * N * P},
        "ssd_chunk_scan": {"bytes": e * b * T * (2 * H * P + 2 * G * N) + 8 * b * T * H + st_in,
                           "flops": int(b * nc * (G * N * Qc * (Qc + 1) + H * P * Qc * (Qc + 1))
                                        + 2 * b * (T - Q) * H * N * P)},
    }


def method_bytes(w) -> int:
    """The bytes the method itself must move with the states kept on chip:
    x, B, C in and y out, dt in, and the final state out."""
    e = 2 if w.dtype == "bf16" else 4
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    return e * b * T * (2 * H * P + 2 * G * N) + 4 * b * T * H + 4 * b * H * N * P


def attainable_peaks(torch, stream) -> dict | None:
    """What the chip delivers to a bare MFMA loop and to a bare streaming copy
    (libssd_peak.so), timed with HIP events on the launch stream, beside the
    datasheet peaks the kernels are reported against."""
    import ctypes

    path = os.path.join(ROOT, "mamba_ssd_scan_04_amd", "libssd_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.ssd_peak_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.ssd_peak_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p]
    lib.ssd_peak_stream_pieces.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    sh = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    blocks, iters = 2048, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def mfma():
        rc = lib.ssd_peak_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), sh)
        if rc != 0:
            raise RuntimeError(f"ssd_peak_mfma_bf16 failed ({rc})")

    t = timed(mfma, 10)
    mfma_tfs = blocks * 4 * iters * 4 * 32768 / t / 1e12
    del out
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)

    def stream_copy():
        rc = lib.ssd_peak_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 nbytes // 16, 16384, sh)
        if rc != 0:
            raise RuntimeError(f"ssd_peak_stream failed ({rc})")

    def stream_pieces():
        rc = lib.ssd_peak_stream_pieces(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                        nbytes // 16, sh)
        if rc != 0:
            raise RuntimeError(f"ssd_peak_stream_pieces failed ({rc})")

    t = timed(stream_copy, 10)
    grid_gbs = 2 * nbytes / t / 1e9
    t = timed(stream_pieces, 10)
    piece_gbs = 2 * nbytes / t / 1e9
    stream_gbs = max(grid_gbs, piece_gbs)
    t = timed(lambda: dst.copy_(src), 10)
    copy_gbs = 2 * nbytes / t / 1e9
    del src, dst
    return {"mfma_bf16_TFLOP/s": round(mfma_tfs, 1), "mfma_bf16_frac_of_peak": round(mfma_tfs / MFMA_BF16_PEAK_TFS, 4),
            "stream_GB/s": round(stream_gbs, 1), "stream_frac_of_peak": round(stream_gbs / HBM_PEAK_GBS, 4),
            "stream_4kb_pieces_GB/s": round(piece_gbs, 1), "stream_grid_stride_GB/s": round(grid_gbs, 1),
            "torch_copy_GB/s": round(copy_gbs, 1),
            "how": "MFMA: 2048 workgroups x 4 waves x 8000 chained v_mfma_f32_32x32x16_bf16; "
                   "stream: the faster of two copies of 1 GiB (read + write) with 16-byte non-temporal vectors, one "
                   "contiguous 4 KB piece per workgroup (262144 workgroups) or grid-stride over 16384 workgroups "
                   "with 4 loads in flight per thread; torch copy_: the same 1 GiB"}


def streams_x(w, state_esz: int) -> bool:
    """The library's copy policy: x (and the chunk scan's carried states) are
    copied non-temporally when the data of one forward (x, y, B, C, dt, cs and
    the inter-chunk states) exceeds the 256 MiB last-level cache."""
    esz = 2 if w.dtype == "bf16" else 4
    bt = w.batch * w.seqlen
    nbytes = (esz * bt * (2 * w.nheads * w.headdim + 2 * w.ngroups * w.dstate) + 8 * bt * w.nheads
              + state_esz * w.batch * w.nchunks * w.nheads * w.headdim * w.dstate)
    return nbytes > 256 * 2**20


def scan_traffic(torch, stream, w, g, cs, states, scan_ms: float, scan_bytes: int) -> dict | None:
    """The chunk scan's memory traffic with none of its arithmetic
    (ssd_peak_scan_traffic in libssd_peak.so: same grid, heads per workgroup,
    block order, copies and stores), timed with HIP events on the launch
    stream: the time its own traffic pattern takes on this GPU, beside the
    kernel's. bf16 inputs and states only."""
    import ctypes

    path = os.path.join(ROOT, "mamba_ssd_scan_04_amd", "libssd_peak.so")
    if not os.path.exists(path) or w.dtype != "bf16" or states.dtype != torch.bfloat16:
        return None
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_peak_scan_traffic.argtypes = [vp] * 8 + [i64] * 9 + [vp]
    nt = streams_x(w, 2)
    # heads per workgroup: the chunk scan's choice (whole rounds of one
    # workgroup per compute unit, C B^T worth about 1.6 heads)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    chunks, hpg = w.batch * w.nchunks * w.ngroups, w.nheads // w.ngroups
    hpw, best = 1, float("inf")
    for h in range(1, min(hpg, 64) + 1):
        nhb = -(-hpg // h)
        cost = -(-chunks * nhb // cus) * (1.6 + -(-hpg // nhb))
        if cost < best - 1e-9:
            hpw, best = h, cost
    nhb = -(-hpg // hpw)
    y2 = torch.empty_like(g["x"])
    sink = torch.empty(w.batch * w.nchunks * w.ngroups * nhb, dtype=torch.float32, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def call():
        rc = lib.ssd_peak_scan_traffic(ptr(g["x"]), ptr(g["B"]), ptr(g["C"]), ptr(states), ptr(g["dt"]), ptr(cs),
                                       ptr(y2), ptr(sink), w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                       w.ngroups, w.chunk_size, hpw, int(nt), ctypes.c_void_p(stream.cuda_stream))
        return rc

    rc = call()
    if rc == -1:
        return None
    if rc != 0:
        raise RuntimeError(f"ssd_peak_scan_traffic failed ({rc})")
    torch.cuda.synchronize()
    if not torch.equal(y2, g["x"]):
        raise RuntimeError("ssd_peak_scan_traffic: y != x")
    for _ in range(5):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del y2, sink
    return {"ms": round(ms, 5), "GB/s": round(scan_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(scan_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "chunk_scan_ms": round(scan_ms, 5), "chunk_scan_over_probe": round(scan_ms / ms, 4),
            "heads_per_workgroup": hpw, "non_temporal_copies": nt,
            "how": "the chunk scan's copies, loads and stores at this shape with no arithmetic (libssd_peak.so "
                   "ssd_peak_scan_traffic); GB/s counts the chunk scan's algorithmic bytes over the probe's time"}


def state_traffic(torch, stream, w, g, state_ms: float, state_bytes: int) -> dict | None:
    """The chunk state's memory traffic with none of its arithmetic
    (ssd_peak_state_traffic in libssd_peak.so: same grid, heads per workgroup,
    block order, 3-deep copy ring, cs and state stores), timed with HIP events
    on the launch stream, beside the kernel's time. bf16 inputs and states
    only."""
    import ctypes

    path = os.path.join(ROOT, "mamba_ssd_scan_04_amd", "libssd_peak.so")
    if not os.path.exists(path) or w.dtype != "bf16":
        return None
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_peak_state_traffic.argtypes = [vp] * 5 + [i64] * 9 + [vp]
    ntc = streams_x(w, 2)
    # heads per workgroup: the chunk state's choice (4 wavefronts; one per head
    # up to 8 output tiles of 32 x 32, halved when the grid would not fill
    # both workgroup slots of every compute unit)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pt, nt = -(-w.headdim // 32), -(-w.dstate // 32)
    wph0 = 1 if pt * nt <= 8 else pt * nt // 8
    hpg = w.nheads // w.ngroups
    hpw = 4 // wph0
    if pt >= 2 * wph0 and w.batch * w.nchunks * w.ngroups * -(-hpg // hpw) < 2 * cus:
        hpw = 4 // (2 * wph0)
    cs2 = torch.empty((w.batch, w.nheads, w.nchunks, w.chunk_size), dtype=torch.float32, device="cuda")
    st2 = torch.empty((w.batch, w.nchunks, w.nheads, w.headdim, w.dstate), dtype=torch.bfloat16, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def call():
        return lib.ssd_peak_state_traffic(ptr(g["x"]), ptr(g["B"]), ptr(g["dt"]), ptr(cs2), ptr(st2), w.batch,
                                          w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size, hpw,
                                          int(ntc), ctypes.c_void_p(stream.cuda_stream))

    rc = call()
    if rc == -1:
        return None
    if rc != 0:
        raise RuntimeError(f"ssd_peak_state_traffic failed ({rc})")
    torch.cuda.synchronize()
    x5 = g["x"].view(w.batch, w.nchunks, w.chunk_size, w.nheads, w.headdim)
    last = x5[:, :, -32:].permute(0, 1, 3, 2, 4)          # [b][c][h][32][P]
    want = last.unsqueeze(3).expand(-1, -1, -1, w.dstate // 32, -1, -1)
    if not torch.equal(st2.view(want.shape), want) or not torch.equal(
            cs2, g["dt"].view(w.batch, w.nchunks, w.chunk_size, w.nheads).permute(0, 3, 1, 2)):
        raise RuntimeError("ssd_peak_state_traffic: wrong copy")
    for _ in range(5):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del cs2, st2
    return {"ms": round(ms, 5), "GB/s": round(state_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(state_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "chunk_state_ms": round(state_ms, 5), "chunk_state_over_probe": round(state_ms / ms, 4),
            "heads_per_workgroup": hpw, "non_temporal_copies": ntc,
            "how": "the chunk state's copies and stores at this shape with no arithmetic (libssd_peak.so "
                   "ssd_peak_state_traffic); GB/s counts the chunk state's algorithmic bytes over the probe's time"}


def source_sha(kernel: str) -> str:
    path = os.path.join(ROOT, "mamba_ssd_scan_04_amd", "csrc", SOURCES[kernel])
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "mamba_ssd_scan_04_amd", "csrc", "ssd_common.hpp")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, state_dtype: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}_{state_dtype}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, w, budget_s: float = 10.0) -> dict:
    """Time the fp64 oracle on a bounded sample of the same workload: whole
    (batch, head) sequences, as many as fit about `budget_s` seconds."""
    import oracle
    from mamba_ssd_scan_04_amd import inputs as gen

    threads = max(1, oracle.default_threads())   # every core in this process's affinity mask
    hpg = w.nheads // w.ngroups

    def run(npairs):
        pairs = [(i // w.nheads, i % w.nheads) for i in range(npairs)]
        # one batch element's heads at a time; the oracle threads over heads
        tot = 0.0
        done = 0
        for bi in sorted({p[0] for p in pairs}):
            hs = [h for (bb, h) in pairs if bb == bi]
            h0, h1 = hs[0], hs[-1] + 1
            g0, g1 = h0 // hpg, (h1 - 1) // hpg + 1
            sl = {"x": inp["x"][bi:bi + 1, :, h0:h1], "dt": inp["dt"][bi:bi + 1, :, h0:h1],
                  "A": inp["A"][h0:h1], "B": inp["B"][bi:bi + 1, :, g0:g1],
                  "C": inp["C"][bi:bi + 1, :, g0:g1], "D": inp["D"][h0:h1]}
            f = gen.to_float64(sl)
            if g1 - g0 > 1 or w.ngroups > 1:
                # map the sliced heads onto their groups explicitly
                idx = [h // hpg - g0 for h in range(h0, h1)]
                f["B"], f["C"] = f["B"][:, :, idx], f["C"][:, :, idx]
            t0 = time.perf_counter()
            oracle.recurrence(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], nthreads=threads)
            tot += time.perf_counter() - t0
            done += h1 - h0
        return tot, done

    probe_pairs = min(threads, w.batch * w.nheads)
    t_probe, _ = run(probe_pairs)
    per_pair = t_probe / probe_pairs * threads  # thread-seconds per pair
    target = int(budget_s * threads / max(per_pair, 1e-9))
    npairs = max(probe_pairs, min(w.batch * w.nheads, target))
    npairs = (npairs // threads) * threads or npairs
    secs, done = run(npairs)
    passes = 1
    # a whole workload shorter than the budget is timed over repeated passes
    while npairs == w.batch * w.nheads and secs < budget_s and passes < 50:
        s2, d2 = run(npairs)
        secs, done, passes = secs + s2, done + d2, passes + 1
    tokens_equiv = done * w.seqlen / w.nheads
    what = (f"{passes} pass(es) over all {npairs}" if passes > 1 else f"{done}")
    # the same on one thread, over one (batch, head) sequence, for the scaling
    f1 = gen.to_float64({"x": inp["x"][:1, :, :1], "dt": inp["dt"][:1, :, :1], "A": inp["A"][:1],
                         "B": inp["B"][:1, :, :1], "C": inp["C"][:1, :, :1], "D": inp["D"][:1]})
    t1 = time.perf_counter()
    oracle.recurrence(f1["x"], f1["dt"], f1["A"], f1["B"], f1["C"], f1["D"], nthreads=1)
    t1 = time.perf_counter() - t1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fc:
            for line in fc:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": tokens_equiv / secs, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity_cpus": oracle.default_threads(),
            "seconds": round(secs, 3), "cpu_model": cpu_model,
            "single_thread_tokens_per_s": round(w.seqlen / w.nheads / t1, 1),
            "sample": f"{what} whole (batch, head) sequences of {w.seqlen} tokens "
                      f"({done / w.nheads:.2f} batch elements' worth of the {w.nheads}-head layer in total), "
                      f"fp64 recurrence in {secs:.2f} s on {threads} threads; tokens/s = sequences*T/H/s"}


def _counter_rows(path: str, counter: str) -> dict:
    """Per kernel name in a rocprofv3 counter_collection.csv: the (dispatch id,
    counter value) pairs, in dispatch order."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: sorted(v) for k, v in rows.items()}


def record_traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, workload, state_dtype) -> int:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of each kernel,
    scaling each counter by what it reads for the 1 GiB copy of
    --calibrate-copy, and write profiles/pmc_<kernel>_<workload>_<state>.json
    tagged with the hash of the kernel source it was taken on.

    The instantiations are told apart by the order in which this script first
    launches them (the profiler prints some template names garbled): for each
    kernel, the first name is ssd_forward with the default state storage
    (bf16 for bf16 inputs), the second ssd_forward with the other storage;
    the gated and then the packed-document instantiations come after both,
    and after them the context-parallel share, whose launches are left out."""
    from mamba_ssd_scan_04_amd import inputs
    nbytes = 1 << 30
    cf = _counter_rows(cal_fetch_csv, "FETCH_SIZE")
    cw = _counter_rows(cal_write_csv, "WRITE_SIZE")
    copy = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        print("no copy kernel in the calibration runs", file=sys.stderr)
        return 1
    mean = lambda v: sum(x[1] for x in v) / len(v)
    f_scale = nbytes / (mean(cf[copy[0]]) * 1024.0)
    w_scale = nbytes / (mean(cw[copy[0]]) * 1024.0)
    fe, wr = _counter_rows(fetch_csv, "FETCH_SIZE"), _counter_rows(write_csv, "WRITE_SIZE")
    w = inputs.WORKLOADS[workload]
    work = kernel_work(w, 2 if state_dtype == "bf16" else 4)
    default = "bf16" if w.dtype == "bf16" else "fp32"
    rank = 0 if state_dtype == default else 1

    for kern in KERNELS:
        names = sorted((k for k in fe if kern + "_kernel" in k), key=lambda k: fe[k][0][0])
        if len(names) <= rank or names[rank] not in wr:
            print(f"{kern}: no dispatch name for {state_dtype} states among {names}", file=sys.stderr)
            continue
        name = names[rank]
        # the packed-document instantiation is the last one launched at full
        # size; later launches of the plain one are the context-parallel
        # share's, on T/8 tokens, and are left out
        last = names[-1] if len(names) > 2 else None
        fsel = [x for x in fe[name] if last is None or x[0] < fe[last][0][0]]
        wsel = [x for x in wr[name] if last is None or last not in wr or x[0] < wr[last][0][0]]
        rd = mean(fsel) * 1024.0 * f_scale
        wb = mean(wsel) * 1024.0 * w_scale
        rec = {"kernel": kern, "dispatch_name": name, "workload": workload, "state_dtype": state_dtype,
               "source_sha": source_sha(kern), "fetch_scale": round(f_scale, 4),
               "write_scale": round(w_scale, 4), "hbm_read_bytes_per_launch": int(rd),
               "hbm_write_bytes_per_launch": int(wb), "hbm_bytes_per_launch": int(rd + wb),
               "alg_bytes_per_launch": work[kern]["bytes"],
               "traffic_over_alg": round((rd + wb) / work[kern]["bytes"], 4)}
        out = os.path.join(ROOT, "profiles", f"pmc_{kern}_{workload}_{state_dtype}.json")
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec), flush=True)
    return 0


def calibrate_copy(torch) -> int:
    """A plain device-to-device copy of a known size: under rocprofv3 --pmc
    FETCH_SIZE / WRITE_SIZE its counters give the scale from counter units to
    bytes (reads and writes of exactly `nbytes` per dispatch)."""
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_dispatch": nbytes,
                      "bytes_written_per_dispatch": nbytes}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed forward calls for this long before the warmup steps, so that the GPU "
                         "clocks have left their idle state whatever --warmup is")
    ap.add_argument("--workload", default="m2p7")
    ap.add_argument("--state-dtype", default=None, choices=["fp32", "bf16"],
                    help="storage of the inter-chunk states (default: bf16 for bf16 inputs); the "
                         "running and final states are fp32 either way")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="(no GPU) write profiles/pmc_*.json from rocprofv3 counter_collection.csv files")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(*args.record_traffic, args.workload, args.state_dtype or "bf16")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import mamba_ssd_scan_04_amd as ssd
    from mamba_ssd_scan_04_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        return calibrate_copy(torch)
    w = inputs.WORKLOADS[args.workload]
    if args.state_dtype is None:
        args.state_dtype = "bf16" if w.dtype == "bf16" else "fp32"
    dev = torch.device("cuda:0")
    inp = inputs.generate(w, seed=0)
    g = {k: v.to(dev) for k, v in inp.items()}
    d = ssd.dims_of(g["x"], g["B"], w.chunk_size, args.state_dtype)
    sbytes = 2 if args.state_dtype == "bf16" else 4
    cs = torch.empty((w.batch, w.nheads, w.nchunks, w.chunk_size), dtype=torch.float32, device=dev)
    states = torch.empty((w.batch, w.nchunks, w.nheads, w.headdim, w.dstate),
                         dtype=torch.bfloat16 if sbytes == 2 else torch.float32, device=dev)
    final = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device=dev)
    y = torch.empty_like(g["x"])
    ws = ssd.alloc_workspace(d, dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    # every timed loop repeats calls whose arguments were checked once
    # (ssd.prepared): the binding's per-call checks take tens of microseconds
    # of host time, more than the small workloads' kernels
    P = ssd.prepared
    stage_calls = [P(ssd.ssd_chunk_cumsum_state, d, g["x"], g["dt"], g["A"], g["B"], cs, states, sh),
                   P(ssd.ssd_state_passing, d, cs, states, final, sh),
                   P(ssd.ssd_chunk_scan, d, g["x"], g["dt"], g["B"], g["C"], g["D"], cs, states, y, sh)]

    def step(ev=None):
        # the launches ssd_forward makes, through the stage entry points, with
        # HIP events between them on the launch stream
        for i, call in enumerate(stage_calls):
            if ev is not None:
                ev[i].record(stream)
            call()
        if ev is not None:
            ev[len(stage_calls)].record(stream)

    forward = P(ssd.ssd_forward, d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y, final, ws, ws.numel(), sh)

    # settle: untimed calls until the clocks have ramped up from idle (input
    # generation on the host leaves the GPU idle for seconds); then the warmup
    # steps, then the timed steps, which run exactly what the warmup ran
    torch.cuda.synchronize()
    settle_calls, ts0 = 0, time.perf_counter()
    while (time.perf_counter() - ts0) * 1e3 < args.settle_ms:
        for _ in range(20):
            forward()
        torch.cuda.synchronize()
        settle_calls += 20
    settle_ms = (time.perf_counter() - ts0) * 1e3
    # the step that is timed: one ssd_forward call
    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        forward()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-call event timings, warm and with the caches cold: between calls a
    # 512 MB scrub buffer (more than the 256 MB last-level cache) is written,
    # outside the timed interval; medians over the calls
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    per_call = {}
    for mode in ("warm", "cold"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for k in range(args.steps):
            if mode == "cold":
                scrub.fill_(k & 0xFF)
            evs[k][0].record(stream)
            forward()
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        per_call[mode] = ts[len(ts) // 2]
    del scrub

    # per-kernel durations: the same launches with events between them
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(KERNELS) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    kms = {name: sum(events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps)) / args.steps
           for i, name in enumerate(KERNELS)}

    # the in-chunk prefix sums alone (ssd_chunk_cumsum, the stage that the
    # forward forms inside the chunk-state launch), for its own HBM rate
    cumsum = P(ssd.ssd_chunk_cumsum, d, g["dt"], g["A"], cs, sh)
    for _ in range(args.warmup):
        cumsum()
    ec0, ec1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ec0.record(stream)
    for _ in range(args.steps):
        cumsum()
    ec1.record(stream)
    torch.cuda.synchronize()
    cum_ms = ec0.elapsed_time(ec1) / args.steps

    # the other storage of the inter-chunk states, same inputs, for reference
    alt = None
    if w.dtype == "bf16":
        alt_sd = "fp32" if args.state_dtype == "bf16" else "bf16"
        d2 = ssd.dims_of(g["x"], g["B"], w.chunk_size, alt_sd)
        ws2 = ssd.alloc_workspace(d2, dev)
        fwd2 = P(ssd.ssd_forward, d2, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], y, final, ws2, ws2.numel(), sh)
        for _ in range(args.warmup):
            fwd2()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            fwd2()
        torch.cuda.synchronize()
        alt_ms = (time.perf_counter() - t2) * 1e3 / args.steps
        alt = {"state_dtype": alt_sd, "ms_per_step": round(alt_ms, 5),
               "tokens_per_s": round(w.batch * w.seqlen / (alt_ms * 1e-3), 1)}
        del ws2

    # the forward with the output gate y * silu(z) fused (ssd_forward_gated)
    zg = inputs.generate_gate(w, seed=1).to(dev)
    yg = torch.empty_like(g["x"])

    gated = P(ssd.ssd_forward_gated, d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, zg, yg, final, ws,
              ws.numel(), sh)

    for _ in range(args.warmup):
        gated()
    torch.cuda.synchronize()
    tg = time.perf_counter()
    for _ in range(args.steps):
        gated()
    torch.cuda.synchronize()
    gated_ms = (time.perf_counter() - tg) * 1e3 / args.steps
    # and the normalisation after the gate (RMSNorm over each token's H*P
    # channels, synthetic weights) in place on the gated output
    wn = torch.randn(w.nheads * w.headdim, generator=torch.Generator().manual_seed(2)).to(dev)
    dn = ssd.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size, w.dtype, "fp32")

    norm = P(ssd.ssd_gated_rmsnorm, dn, yg, None, wn, 1e-5, 1, yg, sh)

    def gated_norm():
        gated()
        norm()

    for _ in range(args.warmup):
        gated_norm()
    torch.cuda.synchronize()
    tn = time.perf_counter()
    for _ in range(args.steps):
        gated_norm()
    torch.cuda.synchronize()
    gated_norm_ms = (time.perf_counter() - tn) * 1e3 / args.steps
    # the normalisation alone (in place, y read and written once)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        norm()
    e1.record(stream)
    torch.cuda.synchronize()
    norm_ms = e0.elapsed_time(e1) / args.steps
    norm_bytes = 2 * yg.numel() * yg.element_size() + 4 * wn.numel()
    del zg, yg, wn

    # packed documents (ssd_forward_varlen): the same rows holding 8 documents
    # each, the state reset at every document start
    seq = inputs.generate_seq_idx(w, 45, 8).to(dev)
    yv = torch.empty_like(g["x"])

    varlen = P(ssd.ssd_forward_varlen, d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, seq, yv, final, ws,
               ws.numel(), sh)

    for _ in range(args.warmup):
        varlen()
    torch.cuda.synchronize()
    tv = time.perf_counter()
    for _ in range(args.steps):
        varlen()
    torch.cuda.synchronize()
    varlen_ms = (time.perf_counter() - tv) * 1e3 / args.steps
    # and with the output gate (ssd_forward_varlen_gated)
    zv = inputs.generate_gate(w, seed=1).to(dev)
    varlen_gated = P(ssd.ssd_forward_varlen_gated, d, g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, seq,
                     zv, yv, final, ws, ws.numel(), sh)
    for _ in range(args.warmup):
        varlen_gated()
    torch.cuda.synchronize()
    tv = time.perf_counter()
    for _ in range(args.steps):
        varlen_gated()
    torch.cuda.synchronize()
    varlen_gated_ms = (time.perf_counter() - tv) * 1e3 / args.steps
    del yv, seq, zv

    # context parallelism as one of 8 GPUs would run it (Knowl 8): its share
    # is T/8 tokens of every row; it runs them from a zero state, forms its
    # total log-decay, folds the 8 shards' boundary states (which the GPUs
    # would all-gather first) and runs its tokens again from its entering state
    K = 8
    Ts = w.seqlen // K
    shard = {k: g[k][:, :Ts].contiguous() for k in ("x", "dt", "B", "C")}
    ds = ssd.dims_of(shard["x"], shard["B"], w.chunk_size, args.state_dtype)
    wss = ssd.alloc_workspace(ds, dev)
    ys = torch.empty_like(shard["x"])
    fins = torch.zeros((K, w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device=dev)
    tots = torch.zeros((K, w.batch, w.nheads), dtype=torch.float32, device=dev)
    ent = torch.empty((K + 1, w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device=dev)

    share_calls = [
        P(ssd.ssd_forward, ds, shard["x"], shard["dt"], g["A"], shard["B"], shard["C"], g["D"], ys, fins[0], wss,
          wss.numel(), sh),
        P(ssd.ssd_total_decay, ds, shard["dt"], g["A"], tots[0], sh),
        P(ssd.ssd_fold_states, ds, K, tots, fins, None, ent, sh),
        P(ssd.ssd_forward_init, ds, shard["x"], shard["dt"], g["A"], shard["B"], shard["C"], g["D"], ent[K - 1], ys,
          fins[0], wss, wss.numel(), sh)]

    def share():
        for call in share_calls:
            call()

    for _ in range(args.warmup):
        share()
    torch.cuda.synchronize()
    tc = time.perf_counter()
    for _ in range(args.steps):
        share()
    torch.cuda.synchronize()
    share_ms = (time.perf_counter() - tc) * 1e3 / args.steps
    cp = {"shards": K, "tokens_per_shard_row": Ts, "share_ms": round(share_ms, 5),
          "what": "one GPU's share of an 8-way context-parallel forward without the all-gather: its T/8 tokens "
                  "from a zero state, its total log-decay, the 8-shard state fold, its tokens again from the "
                  "entering state"}
    del shard, wss, ys, fins, tots, ent

    # the decoding step (ssd_step) at the same layer shape: one token per
    # sequence, the fp32 state read and written in place
    dstep = ssd.make_dims(w.batch, 1, w.nheads, w.headdim, w.dstate, w.ngroups, 32, w.dtype, "fp32")
    sx, sdt = g["x"][:, 0].contiguous(), g["dt"][:, 0].contiguous()
    sB, sC = g["B"][:, 0].contiguous(), g["C"][:, 0].contiguous()
    sstate = torch.zeros((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device=dev)
    sy = torch.empty_like(sx)
    decode_step = P(ssd.ssd_step, dstep, sx, sdt, g["A"], sB, sC, g["D"], sstate, sy, sh)

    for _ in range(args.warmup):
        decode_step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nstep = 200
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(nstep):
        decode_step()
    e1.record(stream)
    torch.cuda.synchronize()
    host_step_us = e0.elapsed_time(e1) * 1e3 / nstep
    # the same steps captured in a HIP graph and replayed, so that the time is
    # the kernels' and not that of launching them one by one from the host
    gstream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gstream):
        captured = P(ssd.ssd_step, dstep, sx, sdt, g["A"], sB, sC, g["D"], sstate, sy, gstream.cuda_stream)
        for _ in range(nstep):
            captured()
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / nstep
    del graph
    esz = 2 if w.dtype == "bf16" else 4
    step_bytes = (2 * 4 * w.batch * w.nheads * w.dstate * w.headdim            # state in and out
                  + 2 * esz * w.batch * w.nheads * w.headdim                   # x, y
                  + 2 * esz * w.batch * w.ngroups * w.dstate + 4 * w.batch * w.nheads)
    decode = {"kernel": "ssd_step", "us_per_step": round(step_us, 2), "us_per_step_host_launched": round(host_step_us, 2),
              "how": f"{nstep} steps captured in one HIP graph and replayed (host-launched: the same steps launched one by one)",
              "tokens_per_s": round(w.batch / (step_us * 1e-6), 1),
              "GB/s": round(step_bytes / (step_us * 1e-6) / 1e9, 1),
              "hbm_frac": round(step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "alg_bytes": step_bytes}

    work = kernel_work(w, sbytes)
    peak_tf = MFMA_BF16_PEAK_TFS if w.dtype == "bf16" else MFMA_F32_PEAK_TFS
    per_kernel = {}
    for name in KERNELS:
        t = kms[name] * 1e-3
        gbs = work[name]["bytes"] / t / 1e9
        tfs = work[name]["flops"] / t / 1e12
        per_kernel[name] = {"ms": round(kms[name], 5), "GB/s": round(gbs, 1),
                            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                            "TFLOP/s": round(tfs, 2), "mfma_frac": round(tfs / peak_tf, 4),
                            "alg_bytes": work[name]["bytes"], "alg_flops": work[name]["flops"]}
    cw = kernel_work(w, sbytes)["ssd_chunk_cumsum"]
    cum_gbs = cw["bytes"] / (cum_ms * 1e-3) / 1e9
    per_kernel["ssd_chunk_cumsum (standalone stage)"] = {
        "ms": round(cum_ms, 5), "GB/s": round(cum_gbs, 1), "hbm_frac": round(cum_gbs / HBM_PEAK_GBS, 4),
        "alg_bytes": cw["bytes"], "note": "formed inside the chunk-state launch in ssd_forward; timed alone here"}
    dom = max(KERNELS, key=lambda n: kms[n])
    traffic = measured_traffic(dom, w.name, args.state_dtype)
    roof = {"kernel": dom, "bound": "hbm", "achieved": per_kernel[dom]["GB/s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": per_kernel[dom]["hbm_frac"], "traffic": traffic}
    tokens = w.batch * w.seqlen
    value = tokens / (ms_per_step * 1e-3)
    mbytes = method_bytes(w)
    dbytes = sum(work[n]["bytes"] for n in KERNELS)
    roof_method = {
        "method_bytes": mbytes, "method_us_at_peak": round(mbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
        "method_frac": round(mbytes / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4),
        "design_bytes": dbytes, "design_us_at_peak": round(dbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
        "design_frac": round(dbytes / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4)}
    peaks = attainable_peaks(torch, stream)
    if peaks is not None:
        peaks["chunk_scan_traffic"] = scan_traffic(torch, stream, w, g, cs, states, kms["ssd_chunk_scan"],
                                                   work["ssd_chunk_scan"]["bytes"])
        peaks["chunk_state_traffic"] = state_traffic(torch, stream, w, g, kms["ssd_chunk_state"],
                                                     work["ssd_chunk_state"]["bytes"])
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "settle": {"ms": round(settle_ms, 1), "calls": settle_calls,
                   "what": "untimed ssd_forward calls before the warmup steps, so that the clocks leave idle"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: Mamba-2 2.7B-layer SSD shape" if w.name == "m2p7" else w.name,
                   "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "ngroups": w.ngroups, "chunk_size": w.chunk_size,
                   "state_dtype": args.state_dtype, "tokens_per_step": tokens},
        "roofline": roof,
        "path_roofline": roof_method,
        "kernels": per_kernel,
        "per_call_ms_median": {"warm": round(per_call["warm"], 5), "cold_cache": round(per_call["cold"], 5),
                               "cold_cache_tokens_per_s": round(tokens / (per_call["cold"] * 1e-3), 1)},
        "attainable_peaks": peaks,
        "evented_ms_per_step": round(staged_ms, 5),
        "other_state_storage": alt,
        "gated": {"entry": "ssd_forward_gated", "ms_per_step": round(gated_ms, 5),
                  "tokens_per_s": round(w.batch * w.seqlen / (gated_ms * 1e-3), 1),
                  "with_rmsnorm_ms_per_step": round(gated_norm_ms, 5),
                  "rmsnorm_alone": {"kernel": "ssd_gated_rmsnorm", "ms": round(norm_ms, 5), "alg_bytes": norm_bytes,
                                    "GB/s": round(norm_bytes / (norm_ms * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(norm_bytes / (norm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                    "how": "in place on the gated output, event-timed on the launch stream"}},
        "varlen": {"entry": "ssd_forward_varlen", "documents_per_row": 8, "ms_per_step": round(varlen_ms, 5),
                   "tokens_per_s": round(w.batch * w.seqlen / (varlen_ms * 1e-3), 1),
                   "with_gate_ms_per_step": round(varlen_gated_ms, 5)},
        "context_parallel": cp,
        "decode": decode,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
