"""Build libssd.so in-tree with hipcc for gfx950.

    python -m mamba_ssd_scan_04_amd.build

Each .hip file is compiled to an object in parallel, then linked into
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
SOURCES = ["ssd_api.hip", "chunk_cumsum.hip", "chunk_state.hip", "state_passing.hip", "chunk_scan.hip",
           "ssd_step.hip", "shard.hip", "norm.hip"]
PEAK_SOURCES = ["peak_probe.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
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
    srcs = SOURCES + PEAK_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], OUT)
    _link([objs[s] for s in PEAK_SOURCES], PEAK_OUT)
    if verbose:
        print(f"built {OUT} and {PEAK_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
