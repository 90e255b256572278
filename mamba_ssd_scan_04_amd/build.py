"""Build libssd.so in-tree with hipcc for gfx950.

    python -m mamba_ssd_scan_04_amd.build

Each .hip file (the chunk-scan unit once per instantiation set) is compiled to
an object in parallel, then linked into
mamba_ssd_scan_04_amd/libssd.so. The attainable-peak probes (an MFMA loop and
a streaming copy, used by the benchmark only) go into libssd_peak.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libssd.so")
PEAK_OUT = os.path.join(PKG, "libssd_peak.so")
BUILD_DIR = os.path.join(PKG, "_build")
ROOT = os.path.dirname(PKG)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]
# (source, object name, extra defines). The chunk-scan kernel is compiled once
# per (input type, state type, variant) from chunk_scan_inst.hip, so that its
# many template instantiations build in parallel.
_SC_UNITS = [("chunk_scan_inst.hip", f"chunk_scan_{x}_{s}_{v}", [f"-DSSD_SC_X={x}", f"-DSSD_SC_S={s}", f"-DSSD_SC_V={v}"])
             for x, s in (("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")) for v in (0, 1, 2, 3)]
SOURCES = [(f, os.path.splitext(f)[0], []) for f in
           ("ssd_api.hip", "chunk_cumsum.hip", "chunk_state.hip", "state_passing.hip", "chunk_scan.hip",
            "ssd_step.hip", "shard.hip", "norm.hip")] + _SC_UNITS
PEAK_SOURCES = [("peak_probe.hip", "peak_probe", [])]


def _compile(unit) -> str:
    src, name, defs = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [HIPCC, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    units = SOURCES + PEAK_SOURCES
    jobs = int(os.environ.get("SSD_BUILD_JOBS", str(min(8, os.cpu_count() or 1))))
    # the chunk-scan units first: they take longest
    order = sorted(units, key=lambda u: u[0] != "chunk_scan_inst.hip")
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(units)))) as ex:
        objs = dict(zip((u[1] for u in order), ex.map(_compile, order)))
    _link([objs[u[1]] for u in SOURCES], OUT)
    _link([objs[u[1]] for u in PEAK_SOURCES], PEAK_OUT)
    if verbose:
        print(f"built {OUT} and {PEAK_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
