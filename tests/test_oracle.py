"""Pins for the fp64 oracle (CPU only).

Nothing here compares the oracle with itself: every check goes against a value
or property the pages or the mathematics fix independently:

* a hand-derived worked example (tests/golden),
* the duality of Knowl 1 (brute-force dual form with explicit mask products),
* closed forms (geometric series, impulse response, a = 1 causal linear
  attention, a = 0 memoryless map, B = 0),
* invariants (linearity, causality, B/C rescaling, group sharing, the reset of
  Knowl 8's variable-length packing),
* the block algorithm of Knowl 2 at many chunk sizes, including Q = 1 (the
  recurrence) and Q = T (the quadratic form), and ragged last chunks,
* planted mistakes: mutated copies of the C oracle must fail the pins.
"""
import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(rng, b, T, H, P, N, G, a_scale=1.0):
    return dict(
        x=rng.standard_normal((b, T, H, P)),
        dt=np.log1p(np.exp(rng.standard_normal((b, T, H)) - 1.0)),
        A=-np.exp(rng.uniform(0.0, np.log(4.0), H)) * a_scale,
        B=rng.standard_normal((b, T, G, N)) / np.sqrt(N),
        C=rng.standard_normal((b, T, G, N)) / np.sqrt(N),
        D=rng.standard_normal(H),
    )


def rec(oracle_mod, inp, **kw):
    return oracle_mod.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], **kw)


def test_golden_hand_example(oracle_mod):
    with open(os.path.join(HERE, "golden", "hand_example_T3.json")) as f:
        g = json.load(f)
    inp = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
    y_ref = np.array(g["expected"]["y"])
    f_ref = np.array(g["expected"]["final"])
    y, fin = rec(oracle_mod, inp)
    np.testing.assert_allclose(y, y_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin, f_ref, rtol=0, atol=1e-12)
    yq = oracle_mod.quadratic(**inp)
    np.testing.assert_allclose(yq, y_ref, rtol=0, atol=1e-12)
    for Q in (1, 2, 3, 4):
        out = oracle_mod.chunked(**inp, Q=Q)
        np.testing.assert_allclose(out["y"], y_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out["final"], f_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 1),
    (1, 5, 2, 3, 2, 1),
    (2, 17, 4, 4, 3, 2),
    (1, 64, 3, 8, 4, 3),
    (2, 33, 4, 2, 5, 4),
])
def test_duality_bruteforce(oracle_mod, shape):
    """Knowl 1: the linear form equals (L o C B^T) X with L as explicit products."""
    rng = np.random.default_rng(sum(shape))
    inp = rand_inputs(rng, *shape)
    y, _ = rec(oracle_mod, inp)
    yq = oracle_mod.quadratic(**inp)
    assert oracle_mod.rel_err(y, yq) < 1e-12


def test_constant_geometric_series(oracle_mod):
    """Constant dt, A, B, C, x: h_t = dt B x^T (1 - a^{t+1}) / (1 - a)."""
    b, T, H, P, N, G = 1, 40, 2, 3, 4, 1
    dt0, A0 = 0.3, np.array([-0.7, -2.0])
    beta = np.linspace(0.5, -0.5, N)
    gamma = np.linspace(-1.0, 1.0, N) + 0.1
    xi = np.array([1.0, -2.0, 0.5])
    D = np.array([0.25, -1.5])
    inp = dict(x=np.broadcast_to(xi, (b, T, H, P)).copy(), dt=np.full((b, T, H), dt0), A=A0,
               B=np.broadcast_to(beta, (b, T, G, N)).copy(),
               C=np.broadcast_to(gamma, (b, T, G, N)).copy(), D=D)
    y, fin = rec(oracle_mod, inp)
    t = np.arange(T)
    for h in range(H):
        a = np.exp(dt0 * A0[h])
        geo = (1 - a ** (t + 1)) / (1 - a)
        y_ref = dt0 * (gamma @ beta) * geo[:, None] * xi[None, :] + D[h] * xi[None, :]
        np.testing.assert_allclose(y[0, :, h, :], y_ref, rtol=1e-13, atol=1e-13)
        fin_ref = dt0 * np.outer(beta, xi) * (1 - a ** T) / (1 - a)
        np.testing.assert_allclose(fin[0, h], fin_ref, rtol=1e-13, atol=1e-13)


def test_impulse_response(oracle_mod):
    """x = e_p at t0: y_t[p] = dt_t0 (C_t.B_t0) exp(sum_{s=t0+1}^{t} dt_s A) for t > t0."""
    rng = np.random.default_rng(3)
    b, T, H, P, N, G = 1, 30, 1, 3, 5, 1
    inp = rand_inputs(rng, b, T, H, P, N, G)
    t0, p = 11, 2
    inp["x"] = np.zeros((b, T, H, P))
    inp["x"][0, t0, 0, p] = 1.0
    y, _ = rec(oracle_mod, inp)
    dt, A, B, C, D = inp["dt"][0, :, 0], inp["A"][0], inp["B"][0, :, 0], inp["C"][0, :, 0], inp["D"][0]
    exp_y = np.zeros(T)
    for t in range(t0, T):
        exp_y[t] = dt[t0] * (C[t] @ B[t0]) * np.exp(A * dt[t0 + 1: t + 1].sum())
    exp_y[t0] += D
    np.testing.assert_allclose(y[0, :, 0, p], exp_y, rtol=1e-12, atol=1e-14)
    other = [q for q in range(P) if q != p]
    assert np.all(y[0, :, 0, other] == 0.0)


def test_no_decay_is_causal_linear_attention(oracle_mod):
    """A = 0 (a = 1): y = tril(C B^T) (dt x) + D x."""
    rng = np.random.default_rng(4)
    b, T, H, P, N, G = 2, 24, 2, 3, 4, 1
    inp = rand_inputs(rng, b, T, H, P, N, G)
    inp["A"] = np.zeros(H)
    y, _ = rec(oracle_mod, inp)
    for bi in range(b):
        for h in range(H):
            att = np.tril(inp["C"][bi, :, 0] @ inp["B"][bi, :, 0].T)
            ref = att @ (inp["dt"][bi, :, h, None] * inp["x"][bi, :, h]) + inp["D"][h] * inp["x"][bi, :, h]
            np.testing.assert_allclose(y[bi, :, h], ref, rtol=1e-12, atol=1e-12)


def test_full_decay_is_memoryless(oracle_mod):
    """dt A <= -800 (a = 0 in fp64): y_t = dt_t (C_t.B_t) x_t + D x_t."""
    rng = np.random.default_rng(5)
    b, T, H, P, N, G = 1, 16, 2, 3, 4, 2
    inp = rand_inputs(rng, b, T, H, P, N, G)
    inp["dt"] = np.full((b, T, H), 2.0)
    inp["A"] = np.array([-400.0, -1000.0])
    y, fin = rec(oracle_mod, inp)
    for h in range(H):
        cb = np.einsum("tn,tn->t", inp["C"][0, :, h], inp["B"][0, :, h])
        ref = (2.0 * cb)[:, None] * inp["x"][0, :, h] + inp["D"][h] * inp["x"][0, :, h]
        np.testing.assert_allclose(y[0, :, h], ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(fin[0, h], 2.0 * np.outer(inp["B"][0, -1, h], inp["x"][0, -1, h]),
                                   rtol=1e-13, atol=1e-13)


def test_zero_B_or_C_gives_skip_only(oracle_mod):
    rng = np.random.default_rng(6)
    inp = rand_inputs(rng, 2, 20, 2, 3, 4, 1)
    for key in ("B", "C"):
        z = dict(inp)
        z[key] = np.zeros_like(inp[key])
        y, fin = rec(oracle_mod, z)
        np.testing.assert_allclose(y, inp["D"][None, None, :, None] * inp["x"], rtol=0, atol=0)
        if key == "B":
            assert np.all(fin == 0.0)


def test_linearity_causality_rescaling(oracle_mod):
    rng = np.random.default_rng(7)
    inp = rand_inputs(rng, 1, 32, 2, 4, 3, 1)
    y0, _ = rec(oracle_mod, inp)
    # linear in x for fixed dt
    x2 = rng.standard_normal(inp["x"].shape)
    y2, _ = rec(oracle_mod, dict(inp, x=x2))
    y12, _ = rec(oracle_mod, dict(inp, x=inp["x"] + 2.5 * x2))
    assert oracle_mod.rel_err(y12, y0 + 2.5 * y2) < 1e-12
    # linear in B (skip term excluded) and in C
    yB, _ = rec(oracle_mod, dict(inp, B=3.0 * inp["B"]))
    skip = inp["D"][None, None, :, None] * inp["x"]
    assert oracle_mod.rel_err(yB - skip, 3.0 * (y0 - skip)) < 1e-12
    # (B, C) -> (s B, C / s) leaves y unchanged
    yS, _ = rec(oracle_mod, dict(inp, B=4.0 * inp["B"], C=inp["C"] / 4.0))
    assert oracle_mod.rel_err(yS, y0) < 1e-12
    # causality: perturbing x at t' leaves y before t' unchanged
    tp = 19
    xp = inp["x"].copy()
    xp[:, tp] += 10.0
    yp, _ = rec(oracle_mod, dict(inp, x=xp))
    assert np.array_equal(yp[:, :tp], y0[:, :tp])
    assert not np.allclose(yp[:, tp:], y0[:, tp:])


def test_group_sharing(oracle_mod):
    """Knowl 7 grouped pattern: G groups with contiguous heads equals G = H with
    B, C replicated per head."""
    rng = np.random.default_rng(8)
    b, T, H, P, N, G = 2, 20, 6, 3, 4, 2
    inp = rand_inputs(rng, b, T, H, P, N, G)
    y, fin = rec(oracle_mod, inp)
    rep = np.arange(H) // (H // G)
    full = dict(inp, B=inp["B"][:, :, rep], C=inp["C"][:, :, rep])
    yf, ff = rec(oracle_mod, full)
    assert np.array_equal(y, yf) and np.array_equal(fin, ff)


def test_reset_splits_sequence(oracle_mod):
    """Knowl 8 variable length: a = 0 at a document start makes the halves independent."""
    rng = np.random.default_rng(9)
    b, T, H, P, N, G = 1, 40, 2, 3, 4, 1
    inp = rand_inputs(rng, b, T, H, P, N, G)
    T1 = 17
    inp["dt"][:, T1] = 2000.0  # exp(2000 * A) == 0 in fp64 for every A <= -1
    y, fin = rec(oracle_mod, inp)
    second = {k: (v[:, T1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y2, fin2 = rec(oracle_mod, second)
    np.testing.assert_allclose(y[:, T1:], y2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(fin, fin2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("T,Qs", [(64, (1, 2, 3, 8, 16, 64, 100)), (37, (1, 5, 8, 16, 32, 37)),
                                  (1, (1, 4))])
def test_chunked_matches_recurrence(oracle_mod, T, Qs):
    """Knowl 2 at many chunk sizes equals Knowl 1's recurrence; Q = 1 is the
    recurrence itself and Q >= T the quadratic form. Also pins the readings of
    'decayed X' (S) and the carried states h_c."""
    rng = np.random.default_rng(T)
    b, H, P, N, G = 2, 4, 3, 5, 2
    inp = rand_inputs(rng, b, T, H, P, N, G, a_scale=0.2)
    for Q in Qs:
        y, fin, snaps = rec(oracle_mod, inp, snap_every=Q)
        out = oracle_mod.chunked(**inp, Q=Q)
        assert oracle_mod.rel_err(out["y"], y) < 1e-12
        assert oracle_mod.rel_err(out["final"], fin) < 1e-12
        assert oracle_mod.rel_err(out["h_in"], snaps) < 1e-12
        # S of chunk c is the final state of the recurrence run on chunk c alone
        nc = -(-T // Q)
        for c in range(nc):
            t0, t1 = c * Q, min(T, (c + 1) * Q)
            part = {k: (v[:, t0:t1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
            _, fc = rec(oracle_mod, part)
            assert oracle_mod.rel_err(out["S"][:, c], fc) < 1e-12
            # cs is the log of the explicit cumulative product of a in the chunk
            a = np.exp(inp["dt"][:, t0:t1] * inp["A"][None, None, :])
            prod = np.cumprod(a, axis=1).transpose(0, 2, 1)
            np.testing.assert_allclose(np.exp(out["cs"][:, :, c, : t1 - t0]), prod, rtol=1e-12)


def test_snapshots_are_entering_states(oracle_mod):
    rng = np.random.default_rng(10)
    inp = rand_inputs(rng, 1, 12, 1, 2, 2, 1)
    _, _, snaps = rec(oracle_mod, inp, snap_every=4)
    assert np.all(snaps[:, 0] == 0.0)
    for c in (1, 2):
        part = {k: (v[:, : 4 * c] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        _, fin = rec(oracle_mod, part)
        np.testing.assert_array_equal(snaps[:, c], fin)


def test_thread_count_does_not_change_results(oracle_mod):
    rng = np.random.default_rng(11)
    inp = rand_inputs(rng, 3, 50, 5, 4, 3, 1)
    y1, f1 = rec(oracle_mod, inp, nthreads=1)
    y8, f8 = rec(oracle_mod, inp, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(f1, f8)


# ---- initial state ("Transformers are SSMs", Knowl 1: the recurrence starts
# from h_{-1}; the pages take it as zero, the library also accepts a given one)

def _split(inp, t0, t1):
    return {k: (v[:, t0:t1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}


def test_initial_state_split_resume(oracle_mod):
    """Running tokens [T1, T) from the state after [0, T1) continues the full
    run exactly: the initial state is the state before the first token."""
    rng = np.random.default_rng(20)
    inp = rand_inputs(rng, 2, 40, 3, 4, 5, 1, a_scale=0.2)
    y, fin = rec(oracle_mod, inp)
    for t1 in (1, 17, 39):
        y1, f1 = rec(oracle_mod, _split(inp, 0, t1))
        y2, f2 = rec(oracle_mod, _split(inp, t1, 40), init=f1)
        assert oracle_mod.rel_err(y2, y[:, t1:]) < 1e-12
        assert oracle_mod.rel_err(f2, fin) < 1e-12
        np.testing.assert_array_equal(y1, y[:, :t1])


def test_initial_state_free_response_closed_form(oracle_mod):
    """With x = 0 the output is the initial state's free decay read out by C:
    y_t = C_t^T exp(A sum_{s<=t} dt_s) h_init, final = exp(A sum_s dt_s) h_init
    (written from the closed form, not from the recurrence)."""
    rng = np.random.default_rng(21)
    b, T, H, P, N, G = 2, 9, 4, 3, 5, 2
    inp = rand_inputs(rng, b, T, H, P, N, G)
    inp["x"] = np.zeros_like(inp["x"])
    init = rng.standard_normal((b, H, N, P))
    y, fin = rec(oracle_mod, inp, init=init)
    hpg = H // G
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            lam = np.cumsum(inp["dt"][bi, :, h]) * inp["A"][h]
            for t in range(T):
                ref = np.exp(lam[t]) * (inp["C"][bi, t, g] @ init[bi, h])
                np.testing.assert_allclose(y[bi, t, h], ref, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(fin[bi, h], np.exp(lam[-1]) * init[bi, h], rtol=1e-13, atol=1e-15)


def test_initial_state_superposition(oracle_mod):
    """The output is affine in the initial state: y(init) - y(0) is the
    free response of init alone (x = 0), for any inputs."""
    rng = np.random.default_rng(22)
    inp = rand_inputs(rng, 1, 21, 2, 4, 3, 1)
    init = rng.standard_normal((1, 2, 3, 4))
    y0, f0 = rec(oracle_mod, inp)
    y1, f1 = rec(oracle_mod, inp, init=init)
    free = dict(inp, x=np.zeros_like(inp["x"]))
    yf, ff = rec(oracle_mod, free, init=init)
    assert oracle_mod.rel_err(y1 - y0, yf) < 1e-11
    assert oracle_mod.rel_err(f1 - f0, ff) < 1e-11


def test_chunked_with_initial_state_matches_recurrence(oracle_mod):
    rng = np.random.default_rng(23)
    inp = rand_inputs(rng, 2, 37, 3, 4, 5, 1, a_scale=0.3)
    init = rng.standard_normal((2, 3, 5, 4))
    y, fin, snaps = rec(oracle_mod, inp, snap_every=8, init=init)
    np.testing.assert_array_equal(snaps[:, 0], init)
    for Q in (1, 5, 8, 37):
        out = oracle_mod.chunked(**inp, Q=Q, init=init)
        assert oracle_mod.rel_err(out["y"], y) < 1e-12
        assert oracle_mod.rel_err(out["final"], fin) < 1e-12
        np.testing.assert_array_equal(out["h_in"][:, 0], init)


def test_initial_state_with_empty_sequence(oracle_mod):
    rng = np.random.default_rng(24)
    inp = rand_inputs(rng, 2, 0, 2, 3, 4, 1)
    init = rng.standard_normal((2, 2, 4, 3))
    y, fin = rec(oracle_mod, inp, init=init)
    assert y.shape == (2, 0, 2, 3)
    np.testing.assert_array_equal(fin, init)


# ---- output gate (Knowl 6: y * SiLU(z))

# ---- variable-length packing ("Transformers are SSMs", Knowl 8: documents
# concatenated into one row, the state reset by a zero decay at each start)

def _random_seq(rng, b, T, ndocs):
    """Non-decreasing ids per row with ndocs - 1 random starts in 1 .. T-1,
    plus a start at t = 1 and two one-token documents at the end."""
    seq = np.zeros((b, T), dtype=np.int32)
    for r in range(b):
        starts = set(rng.choice(np.arange(2, T - 2), size=ndocs - 1, replace=False).tolist())
        starts |= {1, T - 2, T - 1}
        seq[r] = np.cumsum([1 if t in starts else 0 for t in range(T)]) + 7 * r
    return seq


def _documents(seq_row):
    """(start, end) of each document of one row."""
    cuts = [0] + [t for t in range(1, len(seq_row)) if seq_row[t] != seq_row[t - 1]] + [len(seq_row)]
    return list(zip(cuts[:-1], cuts[1:]))


def test_varlen_matches_bruteforce_dual(oracle_mod):
    """The recurrence with resets equals the dual form whose mask products
    take a_s = 0 at every document start (explicit products, no recurrence)."""
    rng = np.random.default_rng(31)
    inp = rand_inputs(rng, 2, 24, 3, 3, 4, 1, a_scale=0.1)
    seq = _random_seq(rng, 2, 24, 4)
    y, _ = rec(oracle_mod, inp, seq_idx=seq)
    assert oracle_mod.rel_err(y, oracle_mod.quadratic(**inp, seq_idx=seq)) < 1e-12


def test_varlen_documents_are_independent(oracle_mod):
    """Each packed document gives what it gives alone from a zero state (the
    first one from the initial state), and the final state is that of the last
    document run alone."""
    rng = np.random.default_rng(32)
    b, T, H, P, N, G = 2, 50, 4, 3, 5, 2
    inp = rand_inputs(rng, b, T, H, P, N, G, a_scale=0.05)
    seq = _random_seq(rng, b, T, 5)
    init = rng.standard_normal((b, H, N, P))
    for ini in (None, init):
        y, fin = rec(oracle_mod, inp, seq_idx=seq, init=ini)
        for r in range(b):
            row = {k: (v[r:r + 1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
            for d, (t0, t1) in enumerate(_documents(seq[r])):
                start = None if (ini is None or d > 0) else ini[r:r + 1]
                yd, fd = rec(oracle_mod, _split(row, t0, t1), init=start)
                assert oracle_mod.rel_err(y[r:r + 1, t0:t1], yd) < 1e-12
            assert oracle_mod.rel_err(fin[r:r + 1], fd) < 1e-12


def test_varlen_one_document_is_the_plain_recurrence(oracle_mod):
    """A row whose ids never change is one sequence: bit-identical results."""
    rng = np.random.default_rng(33)
    inp = rand_inputs(rng, 3, 30, 2, 4, 4, 1)
    seq = np.repeat(np.array([[5], [0], [-3]], dtype=np.int32), 30, axis=1)
    y, fin = rec(oracle_mod, inp, seq_idx=seq)
    y0, fin0 = rec(oracle_mod, inp)
    np.testing.assert_array_equal(y, y0)
    np.testing.assert_array_equal(fin, fin0)


def test_gated_rmsnorm_pins(oracle_mod):
    """The normalisation after the gate (Knowl 6): a constant group maps to the
    weights; with eps = 0 a positive rescaling of y leaves the output unchanged
    and every group of the unweighted output has mean square 1; with one group
    and no gate it is torch's own RMSNorm (a library routine); the gate enters
    as y * silu(z)."""
    import torch

    rng = np.random.default_rng(60)
    b, T, H, P = 2, 5, 3, 4
    y = rng.standard_normal((b, T, H, P))
    z = rng.standard_normal((b, T, H, P))
    w = rng.standard_normal(H * P)
    ones = np.ones(H * P)
    const = np.full((b, T, H, P), 2.5)
    np.testing.assert_allclose(oracle_mod.gated_rmsnorm(const, None, w, 0.0, 3),
                               np.broadcast_to(w.reshape(H, P), (b, T, H, P)), rtol=0, atol=1e-14)
    for groups in (1, 2, 3, 6):
        a = oracle_mod.gated_rmsnorm(y, z, w, 0.0, groups)
        np.testing.assert_allclose(oracle_mod.gated_rmsnorm(7.0 * y, z, w, 0.0, groups), a, rtol=1e-13, atol=1e-13)
        u = oracle_mod.gated_rmsnorm(y, z, ones, 0.0, groups).reshape(b, T, groups, -1)
        np.testing.assert_allclose(np.mean(u * u, axis=-1), 1.0, rtol=1e-13)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y.reshape(b, T, H * P)), (H * P,),
                                       torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle_mod.gated_rmsnorm(y, None, w, 1e-5, 1).reshape(b, T, H * P), ref,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle_mod.gated_rmsnorm(y, z, w, 1e-5, 2),
                               oracle_mod.gated_rmsnorm(oracle_mod.silu_gate(y, z), None, w, 1e-5, 2),
                               rtol=1e-13, atol=1e-13)


def test_silu_gate_identities(oracle_mod):
    """silu(z) = z sigma(z): pinned by sigma(z) + sigma(-z) = 1, i.e.
    silu(z) - silu(-z) = z, by the tanh form z (1 + tanh(z/2)) / 2 (a library
    routine other than exp), and by its limits; the gate is a plain product."""
    z = np.linspace(-30.0, 30.0, 601)
    one = np.ones_like(z)
    s = oracle_mod.silu_gate(one, z)
    np.testing.assert_allclose(s - oracle_mod.silu_gate(one, -z), z, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s, z * (1.0 + np.tanh(z / 2.0)) / 2.0, rtol=1e-12, atol=1e-12)
    assert oracle_mod.silu_gate(1.0, 0.0) == 0.0
    assert abs(oracle_mod.silu_gate(1.0, -800.0)) == 0.0
    assert oracle_mod.silu_gate(1.0, 800.0) == 800.0
    y = np.random.default_rng(25).standard_normal(601)
    np.testing.assert_allclose(oracle_mod.silu_gate(y, z), y * s, rtol=1e-15, atol=0)


MUTANTS = {
    "dropped_skip": ("yt[p] = Dh * xt[p];", "yt[p] = 0.0;"),
    "dropped_dt_input": ("const double u = dtv * Bt[n];", "const double u = Bt[n];"),
    "wrong_decay_sign": ("exp(dtv * Ah)", "exp(-dtv * Ah)"),
    "swapped_B_C": ("const double* Bt = j->B", "const double* Bt = j->C"),
    "wrong_group_map": ("const int64_t g = h / (H / G);", "const int64_t g = h % G;"),
    # y_t read from the state before token t enters it (exclusive mask product)
    "stale_state_output": None,
    # the given initial state ignored (zero start)
    "ignored_initial_state": ("    if (j->init)\n        memcpy(st,", "    if (0)\n        memcpy(st,"),
    # document starts of a packed row not resetting the state
    "ignored_reset": ("starts ? 0.0 : exp(dtv * Ah)", "exp(dtv * Ah)"),
    # the reset taken one token late (at the second token of a document)
    "late_reset": ("const int starts = j->seq && t > 0 && j->seq[b * T + t] != j->seq[b * T + t - 1];",
                   "const int starts = j->seq && t > 1 && j->seq[b * T + t - 1] != j->seq[b * T + t - 2];"),
}

UPDATE_BLOCK = """        for (int64_t n = 0; n < N; ++n) {
            const double u = dtv * Bt[n];
            double* row = st + n * P;
            for (int64_t p = 0; p < P; ++p) row[p] = a * row[p] + u * xt[p];
        }
"""
OUTPUT_BLOCK = """        for (int64_t p = 0; p < P; ++p) yt[p] = Dh * xt[p];
        for (int64_t n = 0; n < N; ++n) {
            const double c = Ct[n];
            const double* row = st + n * P;
            for (int64_t p = 0; p < P; ++p) yt[p] += c * row[p];
        }
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(oracle_mod, name):
    """Each plausible mistake planted in a copy of the C oracle fails a pin."""
    import ctypes

    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "ssd_oracle.c")).read()
    if MUTANTS[name] is None:
        assert UPDATE_BLOCK + OUTPUT_BLOCK in src
        mutated = src.replace(UPDATE_BLOCK + OUTPUT_BLOCK, OUTPUT_BLOCK + UPDATE_BLOCK, 1)
    else:
        old, new = MUTANTS[name]
        assert old in src
        mutated = src.replace(old, new, 1)
    if name == "swapped_B_C":
        mutated = mutated.replace("const double* Ct = j->C", "const double* Ct = j->B", 1)
    tmp = tempfile.mkdtemp()
    try:
        cpath, lpath = os.path.join(tmp, "m.c"), os.path.join(tmp, "libm.so")
        open(cpath, "w").write(mutated)
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", cpath, "-o",
                        lpath, "-lm"], check=True)
        lib = ctypes.CDLL(lpath)
        i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
        lib.ssd_oracle_forward.argtypes = [i64] * 6 + [dp] * 6 + [dp, dp, dp, i64, dp, ctypes.c_int]
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.ssd_oracle_forward_varlen.argtypes = [i64] * 6 + [dp] * 6 + [dp, ip, dp, dp, i64, dp, ctypes.c_int]

        def run_varlen(inp, seq):
            x, dt, A, B, C, D = (np.ascontiguousarray(inp[k], dtype=np.float64)
                                 for k in ("x", "dt", "A", "B", "C", "D"))
            b, T, H, P = x.shape
            y = np.empty_like(x)
            sq = np.ascontiguousarray(seq, dtype=np.int32)
            pp = lambda a: a.ctypes.data_as(dp)
            lib.ssd_oracle_forward_varlen(b, T, H, P, B.shape[3], B.shape[2], pp(x), pp(dt), pp(A), pp(B),
                                          pp(C), pp(D), None, sq.ctypes.data_as(ip), pp(y), None, 0, None, 1)
            return y

        def run(inp, init=None, with_final=False):
            x, dt, A, B, C, D = (np.ascontiguousarray(inp[k], dtype=np.float64)
                                 for k in ("x", "dt", "A", "B", "C", "D"))
            b, T, H, P = x.shape
            y = np.empty_like(x)
            fin = np.empty((b, H, B.shape[3], P))
            pp = lambda a: a.ctypes.data_as(dp)
            ini = None if init is None else pp(np.ascontiguousarray(init, dtype=np.float64))
            lib.ssd_oracle_forward(b, T, H, P, B.shape[3], B.shape[2], pp(x), pp(dt), pp(A),
                                   pp(B), pp(C), pp(D), ini, pp(y), pp(fin), 0, None, 1)
            return (y, fin) if with_final else y

        with open(os.path.join(HERE, "golden", "hand_example_T3.json")) as f:
            g = json.load(f)
        gin = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
        golden_ok = np.allclose(run(gin), np.array(g["expected"]["y"]), rtol=0, atol=1e-12)
        rng = np.random.default_rng(12)
        inp = rand_inputs(rng, 1, 12, 4, 3, 4, 2)
        dual_ok = oracle_mod.rel_err(run(inp), oracle_mod.quadratic(**inp)) < 1e-12
        # split/resume: the second half from the first half's final state
        yfull = run(inp)
        _, f1 = run(_split(inp, 0, 5), with_final=True)
        y2 = run(_split(inp, 5, 12), init=f1)
        resume_ok = oracle_mod.rel_err(y2, yfull[:, 5:]) < 1e-12
        # packed documents: the brute-force dual form with a = 0 at document starts
        seq = np.array([[0, 0, 0, 1, 1, 2, 2, 2, 2, 3, 4, 4]], dtype=np.int32)
        varlen_ok = oracle_mod.rel_err(run_varlen(inp, seq), oracle_mod.quadratic(**inp, seq_idx=seq)) < 1e-12
        assert not (golden_ok and dual_ok and resume_ok and varlen_ok), f"planted mistake {name} was not caught"
    finally:
        shutil.rmtree(tmp)
