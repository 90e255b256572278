"""Seeded synthetic inputs for the SSD chunked forward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it.

Workloads (shapes of Mamba-2 layers, sizes named after the layer they model):

    tiny      b=1 T=256   H=2  P=16 N=16  G=1 Q=64  fp32 x/B/C
    m125      b=4 T=2048  H=24 P=64 N=128 G=1 Q=256 bf16 x/B/C  (125M-layer)
    m2p7      b=8 T=4096  H=80 P=64 N=128 G=1 Q=256 bf16 x/B/C  (2.7B-layer)
    long16k   b=1 T=16384 H=80 P=64 N=128 G=1 Q=256 bf16, dt shift 4
    nsweepN   b=8 T=4096  H=24 P=64 N in {16,64,128,256} G=8 Q=256 bf16

Distributions (all workloads):
    x ~ N(0, 1)                       [b, T, H, P]
    dt = softplus(z - shift), z ~ N(0, 1), shift 2 (4 for long16k)   [b, T, H]
    A_h = -exp(u), u ~ U(0, ln 16)    [H]   (so |A| in [1, 16])
    B, C ~ N(0, 1) / sqrt(N)          [b, T, G, N]
    D_h ~ N(0, 1)                     [H]

Draw order from numpy.random.default_rng(seed): x, z, u, B, C, D. The normal
draws for x, B and C are taken in float32 (numpy's float32 ziggurat), the rest
in float64. dt, A, D are stored as float32; x, B, C as float32 or bfloat16
(round-to-nearest-even through torch). The stored bits are the inputs: the
oracle upcasts them exactly to float64.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    dtype: str  # "fp32" or "bf16": storage type of x, B, C and y
    dt_shift: float = 2.0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        return {
            "workload": self.name, "batch": self.batch, "seqlen": self.seqlen,
            "nheads": self.nheads, "headdim": self.headdim, "dstate": self.dstate,
            "ngroups": self.ngroups, "chunk_size": self.chunk_size,
            "dtype": self.dtype, "dt_shift": self.dt_shift,
        }


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 2, 16, 16, 1, 64, "fp32"),
    "m125": Workload("m125", 4, 2048, 24, 64, 128, 1, 256, "bf16"),
    "m2p7": Workload("m2p7", 8, 4096, 80, 64, 128, 1, 256, "bf16"),
    "long16k": Workload("long16k", 1, 16384, 80, 64, 128, 1, 256, "bf16", 4.0),
    "nsweep16": Workload("nsweep16", 8, 4096, 24, 64, 16, 8, 256, "bf16"),
    "nsweep64": Workload("nsweep64", 8, 4096, 24, 64, 64, 8, 256, "bf16"),
    "nsweep128": Workload("nsweep128", 8, 4096, 24, 64, 128, 8, 256, "bf16"),
    "nsweep256": Workload("nsweep256", 8, 4096, 24, 64, 256, 8, 256, "bf16"),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def _softplus(v: np.ndarray) -> np.ndarray:
    # numerically stable softplus, part of dt's distribution
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def generate(w: Workload, seed: int = 0) -> dict:
    """Draw one seeded input set for workload `w` as CPU torch tensors."""
    rng = np.random.default_rng(seed)
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = rng.standard_normal((b, T, H, P), dtype=np.float32)
    z = rng.standard_normal((b, T, H))
    u = rng.uniform(0.0, math.log(16.0), H)
    Bm = rng.standard_normal((b, T, G, N), dtype=np.float32)
    Cm = rng.standard_normal((b, T, G, N), dtype=np.float32)
    D = rng.standard_normal(H)
    scale = np.float32(1.0 / math.sqrt(N))
    Bm *= scale
    Cm *= scale
    dt = _softplus(z - w.dt_shift).astype(np.float32)
    A = (-np.exp(u)).astype(np.float32)
    dtype = torch_dtype(w.dtype)
    return {
        "x": torch.from_numpy(x).to(dtype),
        "dt": torch.from_numpy(dt),
        "A": torch.from_numpy(A),
        "B": torch.from_numpy(Bm).to(dtype),
        "C": torch.from_numpy(Cm).to(dtype),
        "D": torch.from_numpy(D.astype(np.float32)),
    }


def generate_slow_decay(w: Workload, seed: int = 0) -> dict:
    """Same as `generate`, but with |A| in [1e-3, 1e-1] so that a whole chunk
    decays only by about 0.6-0.99 and the state carried between chunks
    dominates y."""
    inp = generate(w, seed)
    rng = np.random.default_rng(seed + 7919)
    u = rng.uniform(math.log(1e-3), math.log(1e-1), w.nheads)
    inp["A"] = torch.from_numpy((-np.exp(u)).astype(np.float32))
    return inp


def generate_initial_state(w: Workload, seed: int = 0, scale: float = 1.0) -> torch.Tensor:
    """A state to start the recurrence from, [b,H,N,P] fp32: N(0,1) * scale
    (a carried state is a sum of dt-weighted B x^T terms of about this size)."""
    rng = np.random.default_rng(seed + 104729)
    s = rng.standard_normal((w.batch, w.nheads, w.dstate, w.headdim)) * scale
    return torch.from_numpy(s.astype(np.float32))


def generate_gate(w: Workload, seed: int = 0) -> torch.Tensor:
    """The gate branch z [b,T,H,P] for a fused y * silu(z): N(0,1) in x's type."""
    rng = np.random.default_rng(seed + 130363)
    z = rng.standard_normal((w.batch, w.seqlen, w.nheads, w.headdim)).astype(np.float32)
    return torch.from_numpy(z).to(torch_dtype(w.dtype))


def generate_seq_idx(w: Workload, seed: int = 0, docs_per_row: int = 4, cuts=()) -> torch.Tensor:
    """Document ids [b,T] int32 for rows that pack several documents: per row,
    docs_per_row - 1 document starts drawn uniformly from 1 .. T-1 without
    repetition, plus the starts listed in `cuts` (those inside the row); ids
    count the starts so far plus 1000 * row (they never decrease along T)."""
    rng = np.random.default_rng(seed + 15485863)
    b, T = w.batch, w.seqlen
    ids = np.zeros((b, T), dtype=np.int32)
    for r in range(b):
        k = min(max(docs_per_row - 1, 0), max(T - 1, 0))
        starts = set(rng.choice(np.arange(1, T), size=k, replace=False).tolist()) if k > 0 else set()
        starts |= {int(c) for c in cuts if 0 < c < T}
        flags = np.zeros(T, dtype=np.int32)
        flags[sorted(starts)] = 1
        ids[r] = np.cumsum(flags) + 1000 * r
    return torch.from_numpy(ids)


def to_float64(inp: dict) -> dict:
    """Exact upcast of the stored bits to float64 numpy arrays."""
    return {k: v.float().numpy().astype(np.float64) for k, v in inp.items()}
