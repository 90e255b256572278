"""fp64 CPU oracle for the SSD chunked forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the library and its Python binding never do.
It shares no code with the HIP path. All sources: "Transformers are SSMs"
(Dao & Gu), as summarised on the chapterpal page (Knowls 1, 2 and 7).

Three forms of the same map, in float64:

* `recurrence`  - the linear (recurrent) form of Knowl 1, in plain C
                  (ssd_oracle.c). This is the oracle the HIP path is judged by.
* `quadratic`   - the dual (quadratic attention) form of Knowl 1, built by brute
                  force with the mask entries as explicit products. A pin for
                  `recurrence` at small T.
* `chunked`     - the block-decomposition algorithm of Knowl 2 in its own step
                  order, returning its intermediates (chunk cumulative decay,
                  chunk states, carried states). Stage reference for the HIP
                  kernels; pinned against `recurrence` by chunk-size invariance.

Discretisation (not on the pages; the plainest reading the rest supports):
a_t = exp(dt_t * A_h), the input term is dt_t * B_t x_t^T, and a skip term
D_h * x_t is added to y.

Parity: `recurrence` is pinned by `quadratic` (duality, Knowl 1), closed forms
and a hand-derived example; `chunked` is pinned by `recurrence`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c with gcc (-O2, IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
             _SRC, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
        lib.ssd_oracle_forward.argtypes = [i64] * 6 + [dp] * 6 + [dp, dp, dp, i64, dp, ctypes.c_int]
        lib.ssd_oracle_forward.restype = ctypes.c_int
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.ssd_oracle_forward_varlen.argtypes = ([i64] * 6 + [dp] * 6 + [dp, ip, dp, dp, i64, dp,
                                                                          ctypes.c_int])
        lib.ssd_oracle_forward_varlen.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def recurrence(x, dt, A, B, C, D, snap_every: int = 0, nthreads: int | None = None, init=None,
               seq_idx=None):
    """Knowl 1 linear form, fp64. Returns (y, final[, snaps]).

    x [b,T,H,P], dt [b,T,H], A [H], B/C [b,T,G,N], D [H] (any float arrays;
    converted to contiguous float64). final is [b,H,N,P]. init [b,H,N,P] is
    the state before the first token (None: zero). With snap_every=Q, also
    returns snaps [b,nc,H,N,P]: the state entering each chunk of Q tokens.
    seq_idx [b,T] (integer, non-decreasing along T) packs several documents
    into one row (Knowl 8): the decay is 0 at each token whose id differs from
    the previous token's, which drops the state entering that document.
    """
    x, dt, A, B, C, D = (np.ascontiguousarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    if init is not None:
        init = np.ascontiguousarray(init, dtype=np.float64)
    if seq_idx is not None:
        seq_idx = np.ascontiguousarray(seq_idx, dtype=np.int32)
        if seq_idx.shape != x.shape[:2]:
            raise ValueError(f"seq_idx must be [b,T] = {x.shape[:2]}, got {seq_idx.shape}")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty_like(x)
    final = np.empty((b, H, N, P))
    snaps = None
    if snap_every > 0:
        nc = -(-T // snap_every)
        snaps = np.empty((b, nc, H, N, P))
    if init is not None and init.shape != (b, H, N, P):
        raise ValueError(f"init must be [b,H,N,P] = {(b, H, N, P)}, got {init.shape}")
    sp = None if seq_idx is None else seq_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = _load().ssd_oracle_forward_varlen(b, T, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                           _ptr(C), _ptr(D), _ptr(init), sp, _ptr(y), _ptr(final),
                                           snap_every, _ptr(snaps), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_forward failed with code {rc}")
    return (y, final, snaps) if snap_every > 0 else (y, final)


def _heads_to_groups(H, G):
    return np.arange(H) // (H // G)


def quadratic(x, dt, A, B, C, D, seq_idx=None):
    """Knowl 1 dual form by brute force: Y = (L o C B^T) (dt*x) + D x.

    L[t, i] is formed as the explicit product a_{i+1} * ... * a_t for t >= i
    (the empty product, 1, on the diagonal) and 0 above it. With seq_idx, a_s
    is 0 at every document start s (Knowl 8). O(T^3) per head: for small T
    only.
    """
    x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    b, T, H, P = x.shape
    gid = _heads_to_groups(H, B.shape[2])
    y = np.empty_like(x)
    for bi in range(b):
        for h in range(H):
            g = gid[h]
            a = np.exp(dt[bi, :, h] * A[h])
            if seq_idx is not None:
                sq = np.asarray(seq_idx)[bi]
                a[1:][sq[1:] != sq[:-1]] = 0.0
            Lm = np.zeros((T, T))
            for t in range(T):
                for i in range(t + 1):
                    prod = 1.0
                    for s in range(i + 1, t + 1):
                        prod *= a[s]
                    Lm[t, i] = prod
            gram = C[bi, :, g, :] @ B[bi, :, g, :].T        # [T, T]: C_t . B_i
            xin = dt[bi, :, h][:, None] * x[bi, :, h, :]     # dt-scaled input
            y[bi, :, h, :] = (Lm * gram) @ xin + D[h] * x[bi, :, h, :]
    return y


def chunked(x, dt, A, B, C, D, Q: int, init=None):
    """Knowl 2 block decomposition in fp64, steps in the pages' order.

    Returns a dict:
      y      [b,T,H,P]   output
      final  [b,H,N,P]   final state h_{T/Q}
      cs     [b,H,nc,Q]  in-chunk inclusive prefix sums of dt*A (log of the
                         cumulative products); entries past a ragged chunk's
                         end are NaN
      S      [b,nc,H,N,P] chunk states: B^T applied to the chunk's dt-scaled
                         inputs after their decay (step 2 of the decomposition)
      h_in   [b,nc,H,N,P] state entering each chunk (h_c; h_0 = init, zero if None)
    Reading of the decay in step 2: token j of a chunk is weighted by the decay
    from j to the chunk's end, a_{j+1} ... a_{Q-1}; of the decay of the entering
    state in step 4: row j is scaled by a_0 ... a_j. A last chunk shorter than
    Q is allowed.
    """
    x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    gid = _heads_to_groups(H, G)
    nc = -(-T // Q)
    ell = dt * A[None, None, :]                               # log a_t, [b,T,H]
    xin = dt[..., None] * x                                   # dt-scaled X
    Bh = B[:, :, gid, :]                                      # [b,T,H,N]
    Ch = C[:, :, gid, :]
    cs_out = np.full((b, H, nc, Q), np.nan)
    S = np.zeros((b, nc, H, N, P))
    y = np.empty_like(x)
    seg = []
    # step 1-2: partition, in-chunk cumulative decay (log space)
    for c in range(nc):
        t0, t1 = c * Q, min((c + 1) * Q, T)
        cs = np.cumsum(ell[:, t0:t1, :], axis=1)              # [b,Qc,H]
        cs_out[:, :, c, : t1 - t0] = cs.transpose(0, 2, 1)
        seg.append((t0, t1, cs))
    # step 3: per chunk, diagonal block and right-factor chunk state
    for c, (t0, t1, cs) in enumerate(seg):
        csh = cs.transpose(0, 2, 1)                           # [b,H,Qc]
        diff = csh[:, :, :, None] - csh[:, :, None, :]        # cs_j - cs_i
        Qc = t1 - t0
        lower = np.tril(np.ones((Qc, Qc), dtype=bool))
        Lmask = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        gram = np.einsum("bjhn,bihn->bhji", Ch[:, t0:t1], Bh[:, t0:t1])
        y[:, t0:t1] = np.einsum("bhji,bihp->bjhp", Lmask * gram, xin[:, t0:t1])
        w = np.exp(csh[:, :, -1:] - csh)                      # decay to chunk end
        S[:, c] = np.einsum("bhj,bjhn,bjhp->bhnp", w, Bh[:, t0:t1], xin[:, t0:t1])
    # step 4: inter-chunk recurrence on chunk states
    h_in = np.zeros((b, nc, H, N, P))
    state = np.zeros((b, H, N, P)) if init is None else np.array(init, dtype=np.float64)
    for c, (t0, t1, cs) in enumerate(seg):
        h_in[:, c] = state
        state = np.exp(cs[:, -1, :])[:, :, None, None] * state + S[:, c]
    # step 5: off-diagonal output from the incoming state, combine, skip term
    for c, (t0, t1, cs) in enumerate(seg):
        ydec = np.exp(cs)                                     # a_0 ... a_j, [b,Qc,H]
        y[:, t0:t1] += ydec[..., None] * np.einsum("bjhn,bhnp->bjhp", Ch[:, t0:t1], h_in[:, c])
    y += D[None, None, :, None] * x
    return {"y": y, "final": state, "cs": cs_out, "S": S, "h_in": h_in}


def silu_gate(y, z):
    """The Mamba-2 block's output gate ("Transformers are SSMs", Knowl 6, the
    SiLU(z) branch applied to the SSD output), fp64: y * silu(z) with
    silu(z) = z / (1 + exp(-z)), elementwise."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return y * (z / (1.0 + np.exp(-z)))


def gated_rmsnorm(y, z, weight, eps: float, groups: int = 1):
    """The normalisation after the gate in the Mamba-2 block ("Transformers are
    SSMs", Knowl 6: Y_g = Y * SiLU(z), then a group or RMS norm before the
    output projection), fp64. Per token, the e*d = H*P channels of y [b,T,H,P]
    are cut into `groups` equal contiguous groups (1: plain RMSNorm over all
    channels; Knowl 8's GroupNorm with groups divisible by the TP degree), and
    each group is divided by its root mean square:
        g   = y * silu(z)   (y itself when z is None)
        out = g / sqrt(mean over the group of g^2 + eps) * weight[channel]
    weight is [H*P]."""
    y = np.asarray(y, dtype=np.float64)
    g = y if z is None else silu_gate(y, z)
    b, T, H, P = g.shape
    C = H * P
    if C % groups != 0:
        raise ValueError("groups must divide H*P")
    v = g.reshape(b, T, groups, C // groups)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    out = (v / np.sqrt(ms + eps)).reshape(b, T, C) * np.asarray(weight, dtype=np.float64)[None, None, :]
    return out.reshape(b, T, H, P)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (0 when both are all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
