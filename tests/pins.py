"""Pins of the fp64 oracle: checks against what the pages print and what mathematics fixes.

Each pin takes an oracle instance (so the mutation test can run them on deliberately broken
builds) and raises AssertionError when the oracle disagrees. None of them re-types the oracle's
own formulas: ZOH is re-derived through the matrix exponential of the augmented system (Van Loan),
the LTI case through the convolution kernel K̄, the selective case through a brute-force unroll of
the time-varying products, and associativity through random tree-ordered affine compositions.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.linalg
from scipy.special import expit

from conftest import read_golden


# ---------------------------------------------------------------------------------------------
# Independent constructions
# ---------------------------------------------------------------------------------------------
def zoh_vanloan(a_diag, b_vec, delta):
    """Exact ZOH of h' = diag(a) h + b x with x held over [0, Δ]:
    expm([[ΔA, Δb], [0, 0]]) = [[Ā, B̄], [0, 1]] (Van Loan's block exponential)."""
    a_diag = np.asarray(a_diag, dtype=np.float64)
    N = a_diag.shape[0]
    M = np.zeros((N + 1, N + 1))
    M[:N, :N] = np.diag(a_diag) * delta
    M[:N, N] = np.asarray(b_vec, dtype=np.float64) * delta
    E = scipy.linalg.expm(M)
    return E[:N, :N], E[:N, N]


def silu_lib(v):
    return v * expit(v)


def _close(got, want, rtol=1e-11, atol=1e-12, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


def _golden_pairs(name):
    out = {}
    for row in read_golden(name):
        if len(row) == 2:
            out[row[0]] = float(row[1])
    return out


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------------------------
def pin_scalar_worked_example(orc):
    """kasblo page, scalar example: Ā, B̄ and the four printed impulse weights."""
    g = _golden_pairs("kasblo_scalar_example.txt")
    half = 0.5 * 10.0 ** (-g["printed_decimals"])
    abar, bcoef = orc.zoh(g["delta"], g["A"])
    bbar = bcoef * g["B"]
    assert abs(abar - g["abar"]) <= half, abar
    assert abs(bbar - g["bbar"]) <= half, bbar
    # the page's closed forms: Ā = e^{-1/2}, B̄ = 1 - e^{-1/2}
    _close(abar, math.exp(-0.5), what="abar closed form")
    _close(bbar, 1.0 - math.exp(-0.5), what="bbar closed form")
    L = 8
    x = np.zeros((1, 1, L)); x[0, 0, 0] = 1.0
    y, _ = orc.scan_fwd(x, np.full((1, 1, L), g["delta"]), [[g["A"]]], np.full((1, L, 1), g["B"]),
                        np.full((1, L, 1), g["C"]), D=[g["D"]])
    for k in range(4):
        assert abs(y[0, 0, k] - g[f"weight_lag{k}"]) <= half, (k, y[0, 0, k])
    # unrolled closed form: y_k = B̄ Ā^k for an impulse (C = 1)
    _close(y[0, 0], (1.0 - math.exp(-0.5)) * np.exp(-0.5 * np.arange(L)), what="impulse response")


def pin_delta_gate(orc):
    """kasblo page, Δ as a gate: printed retention for Δ = 0.1 and Δ = 2 at A = -1."""
    rows = read_golden("kasblo_delta_gate.txt")
    hdr = {r[0]: float(r[1]) for r in rows if len(r) == 2}
    half = 0.5 * 10.0 ** (-hdr["printed_decimals"])
    cases = [(float(r[1]), float(r[3])) for r in rows if len(r) == 4 and r[0] == "delta"]
    assert len(cases) == 2
    for dlt, printed in cases:
        abar, _ = orc.zoh(dlt, hdr["A"])
        assert abs(abar - printed) <= half, (dlt, abar)
        _close(abar, math.exp(-dlt), what="retention closed form")


def pin_decay_impulse(orc):
    """sharin page §①: an impulse under decay 0.8 has all but vanished 50 steps later (0.8^50)."""
    g = _golden_pairs("sharin_scan_properties.txt")
    r, steps = g["decay"], int(g["steps"])
    A = math.log(r)
    B = A / (r - 1.0)  # makes B̄ = (r - 1)/A · B = 1
    L = steps + 1
    x = np.zeros((1, 1, L)); x[0, 0, 0] = 1.0
    y, h = orc.scan_fwd(x, np.ones((1, 1, L)), [[A]], np.full((1, L, 1), B), np.ones((1, L, 1)),
                        D=[0.0])
    _close(y[0, 0], r ** np.arange(L), rtol=1e-12, what="0.8^t")
    assert y[0, 0, steps] / y[0, 0, 0] < 1e-4
    _close(h[0, 0, 0], r ** steps, rtol=1e-12, what="state after 50 steps")


def pin_cumulative_sum(orc):
    """sharin page §①: discrete a = 1 accumulates; here the continuous limit A = 0."""
    L = 128
    rng = _rng(11)
    x = rng.integers(-8, 9, size=(1, 1, L)).astype(np.float64)
    y, h = orc.scan_fwd(x, np.ones((1, 1, L)), [[0.0]], np.ones((1, L, 1)), np.ones((1, L, 1)),
                        D=[0.0])
    assert np.array_equal(y[0, 0], np.cumsum(x[0, 0])), "A = 0 must give the exact running sum"
    assert h[0, 0, 0] == np.sum(x)


def pin_lti_convolution(orc):
    """Time-invariant Δ, B, C: the scan equals y = x * K̄ + D x with K̄_k = C Ā^k B̄
    ("State Space Models（SSM）とMamba" §2.3; kasblo page, recurrence vs convolution section)."""
    rng = _rng(3)
    b, d, N, L = 2, 2, 4, 16
    A = -rng.uniform(0.2, 2.0, size=(d, N)); A[1, 2] = 0.0
    dl = rng.uniform(0.05, 0.8, size=(b, d))
    Bv = rng.normal(size=(b, N)); Cv = rng.normal(size=(b, N)); D = rng.normal(size=d)
    x = rng.normal(size=(b, d, L))
    delta = np.repeat(dl[:, :, None], L, axis=2)
    B = np.repeat(Bv[:, None, :], L, axis=1); C = np.repeat(Cv[:, None, :], L, axis=1)
    y, _ = orc.scan_fwd(x, delta, A, B, C, D=D)
    want = np.empty_like(y)
    for ib in range(b):
        for idd in range(d):
            Ab, Bb = zoh_vanloan(A[idd], Bv[ib], dl[ib, idd])
            K = np.array([Cv[ib] @ np.linalg.matrix_power(Ab, k) @ Bb for k in range(L)])
            want[ib, idd] = np.convolve(x[ib, idd], K)[:L] + D[idd] * x[ib, idd]
    _close(y, want, what="LTI convolution")


def pin_selective_unroll(orc):
    """Time-varying Δ_t, B_t, C_t: brute-force unroll y_t = Σ_{s<=t} C_t (Π_{r=s+1..t} Ā_r) B̄_s x_s + D x_t."""
    rng = _rng(5)
    b, d, N, L = 2, 3, 5, 12
    A = -rng.uniform(0.1, 3.0, size=(d, N)); A[2, 0] = 0.0
    delta = rng.uniform(0.01, 1.5, size=(b, d, L))
    B = rng.normal(size=(b, L, N)); C = rng.normal(size=(b, L, N)); D = rng.normal(size=d)
    x = rng.normal(size=(b, d, L))
    y, h = orc.scan_fwd(x, delta, A, B, C, D=D)
    want_y = np.empty_like(y)
    want_h = np.empty_like(h)
    for ib in range(b):
        for idd in range(d):
            Abars, Bbars = zip(*[zoh_vanloan(A[idd], B[ib, t], delta[ib, idd, t]) for t in range(L)])
            for t in range(L + 1):
                hs = np.zeros(N)
                for s in range(min(t + 1, L)):
                    P = np.eye(N)
                    for r in range(s + 1, min(t + 1, L)):
                        P = Abars[r] @ P
                    hs = hs + P @ Bbars[s] * x[ib, idd, s]
                if t < L:
                    want_y[ib, idd, t] = C[ib, t] @ hs + D[idd] * x[ib, idd, t]
                else:
                    want_h[ib, idd] = hs
    _close(y, want_y, what="selective unroll y")
    _close(h, want_h, what="selective unroll final state")


def pin_closed_gate(orc):
    """sharin page §②: a closed gate (B_t = 0) lets the state only decay, by Π Ā_t = exp(A Σ Δ_t)."""
    rng = _rng(7)
    b, d, N, t0, t1 = 1, 2, 3, 9, 20
    A = -rng.uniform(0.1, 1.0, size=(d, N))
    delta = rng.uniform(0.05, 0.5, size=(b, d, t1))
    B = rng.normal(size=(b, t1, N)); B[:, t0:, :] = 0.0
    C = rng.normal(size=(b, t1, N)); x = rng.normal(size=(b, d, t1))
    _, h_at = orc.scan_fwd(x[:, :, :t0], delta[:, :, :t0], A, B[:, :t0], C[:, :t0])
    _, h_end = orc.scan_fwd(x, delta, A, B, C)
    decay = np.exp(A[None, :, :] * delta[:, :, t0:].sum(axis=2)[:, :, None])
    _close(h_end, decay * h_at, what="closed-gate decay")


def pin_delta_limits(orc):
    """Δ -> 0 keeps the state (Ā = 1, B̄ = 0); Δ -> ∞ with A < 0 writes the input (h -> -B x / A)."""
    rng = _rng(9)
    b, d, N = 2, 3, 4
    A = -rng.uniform(0.5, 2.0, size=(d, N))
    st = rng.normal(size=(b, d, N)); x = rng.normal(size=(b, d))
    B = rng.normal(size=(b, N)); C = rng.normal(size=(b, N)); D = rng.normal(size=d)
    y, st2 = orc.scan_step(st, x, np.zeros((b, d)), A, B, C, D=D)
    assert np.array_equal(st2, st), "Δ = 0 must leave the state untouched"
    _close(y, np.einsum("bn,bdn->bd", C, st) + D[None, :] * x, what="Δ = 0 readout")
    _, st3 = orc.scan_step(st, x, np.full((b, d), 200.0), A, B, C)
    _close(st3, -B[:, None, :] * x[:, :, None] / A[None, :, :], rtol=1e-12, what="Δ -> ∞ state")


def pin_affine_associativity(orc):
    """kasblo page, selective-scan section: (A2,b2)∘(A1,b1) = (A2A1, A2b1 + b2) is associative, so any
    tree order of the per-step maps gives the sequential state; chaining calls through h0 is one
    such order (segments carried across calls)."""
    rng = _rng(13)
    b, d, N, L = 1, 2, 3, 33
    A = -rng.uniform(0.05, 1.5, size=(d, N))
    delta = rng.uniform(0.01, 0.9, size=(b, d, L))
    B = rng.normal(size=(b, L, N)); C = rng.normal(size=(b, L, N)); x = rng.normal(size=(b, d, L))
    D = rng.normal(size=d); z = rng.normal(size=(b, d, L))
    y, h = orc.scan_fwd(x, delta, A, B, C, D=D, z=z)
    for idd in range(d):
        maps = []
        for t in range(L):
            Ab, Bb = zoh_vanloan(A[idd], B[0, t], delta[0, idd, t])
            maps.append((np.diag(Ab).copy(), Bb * x[0, idd, t]))
        for trial in range(4):
            items = list(maps)
            while len(items) > 1:  # random adjacent merges = a random parenthesisation
                i = int(rng.integers(0, len(items) - 1))
                (a1, b1), (a2, b2) = items[i], items[i + 1]
                items[i:i + 2] = [(a2 * a1, a2 * b1 + b2)]
            _close(items[0][1], h[0, idd], what=f"tree order {trial}")
    cuts = [0, 5, 6, 20, L]
    hc = None
    ys = []
    for s, e in zip(cuts[:-1], cuts[1:]):
        yy, hc = orc.scan_fwd(x[:, :, s:e], delta[:, :, s:e], A, B[:, s:e], C[:, s:e], D=D,
                              z=z[:, :, s:e], h0=hc)
        ys.append(yy)
    _close(np.concatenate(ys, axis=2), y, what="chained segments y")
    _close(hc, h, what="chained segments state")


def pin_prefill_equals_decode(orc):
    """Training/prefill and recurrent decode compute the same map (kasblo page, prefill vs decode)."""
    rng = _rng(17)
    b, d, N, L = 2, 3, 4, 10
    A = -rng.uniform(0.1, 2.0, size=(d, N))
    delta = rng.uniform(0.01, 1.0, size=(b, d, L))
    B = rng.normal(size=(b, L, N)); C = rng.normal(size=(b, L, N)); x = rng.normal(size=(b, d, L))
    D = rng.normal(size=d); z = rng.normal(size=(b, d, L))
    y, h = orc.scan_fwd(x, delta, A, B, C, D=D, z=z)
    st = np.zeros((b, d, N))
    for t in range(L):
        yt, st = orc.scan_step(st, x[:, :, t], delta[:, :, t], A, B[:, t], C[:, t], D=D, z=z[:, :, t])
        _close(yt, y[:, :, t], what=f"decode step {t}")
    _close(st, h, what="decode final state")


def pin_skip_and_gate(orc):
    """C = 0 leaves only the skip D·x, times silu(z) from the gate; z = 0 closes the output exactly."""
    rng = _rng(19)
    b, d, N, L = 2, 3, 4, 9
    A = -rng.uniform(0.1, 2.0, size=(d, N))
    delta = rng.uniform(0.01, 1.0, size=(b, d, L))
    B = rng.normal(size=(b, L, N)); x = rng.normal(size=(b, d, L)); D = rng.normal(size=d)
    z = 3.0 * rng.normal(size=(b, d, L))
    y, _ = orc.scan_fwd(x, delta, A, B, np.zeros((b, L, N)), D=D, z=z)
    _close(y, D[None, :, None] * x * silu_lib(z), what="skip times silu gate")
    C = rng.normal(size=(b, L, N))
    y0, _ = orc.scan_fwd(x, delta, A, B, C, D=D, z=np.zeros((b, d, L)))
    assert np.all(y0 == 0.0)
    ynog, _ = orc.scan_fwd(x, delta, A, B, C, D=D)
    yg, _ = orc.scan_fwd(x, delta, A, B, C, D=D, z=z)
    _close(yg, ynog * silu_lib(z), what="gate multiplies the SSM output")


def pin_linearity(orc):
    """With the gate off the map x -> y is linear (the recurrence is linear in x)."""
    rng = _rng(23)
    b, d, N, L = 1, 2, 3, 15
    A = -rng.uniform(0.1, 2.0, size=(d, N))
    delta = rng.uniform(0.01, 1.0, size=(b, d, L))
    B = rng.normal(size=(b, L, N)); C = rng.normal(size=(b, L, N)); D = rng.normal(size=d)
    x1 = rng.normal(size=(b, d, L)); x2 = rng.normal(size=(b, d, L))
    y1, _ = orc.scan_fwd(x1, delta, A, B, C, D=D)
    y2, _ = orc.scan_fwd(x2, delta, A, B, C, D=D)
    y12, _ = orc.scan_fwd(2.0 * x1 - 0.5 * x2, delta, A, B, C, D=D)
    _close(y12, 2.0 * y1 - 0.5 * y2, rtol=1e-10, atol=1e-12, what="linearity in x")


# ---------------------------------------------------------------------------------------------
# Gradients: the backward oracle against finite differences of the (pinned) forward oracle, and
# closed forms. The pages define only the forward map; its derivatives are fixed by it.
# ---------------------------------------------------------------------------------------------
def _loss(orc, inp, dy, dhf):
    y, h = orc.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp.get("D"), z=inp.get("z"),
                        h0=inp.get("h0"))
    return float(np.sum(dy * y) + np.sum(dhf * h))


def _fd_check(orc, inp, dy, dhf, names, rtol=2e-6, atol=1e-8, only=None):
    g = orc.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp.get("D"), z=inp.get("z"),
                     h0=inp.get("h0"), dy=dy, dh_final=dhf)
    key = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz", "h0": "dh0"}
    for name in names:
        arr = inp[name]
        num = np.zeros_like(arr)
        idx_list = list(np.ndindex(arr.shape)) if only is None or name not in only else only[name]
        for idx in idx_list:
            v = arr[idx]
            eps = 1e-6 * max(1.0, abs(v))
            arr[idx] = v + eps
            lp = _loss(orc, inp, dy, dhf)
            arr[idx] = v - eps
            lm = _loss(orc, inp, dy, dhf)
            arr[idx] = v
            num[idx] = (lp - lm) / (2 * eps)
        got = g[key[name]]
        sel = tuple(np.array(idx_list).T) if idx_list else ()
        _close(got[sel], num[sel], rtol=rtol, atol=atol, what=f"d{name} vs finite differences")
    return g


def pin_bwd_finite_differences(orc):
    """Every gradient (x, Δ, A, B, C, D, z, initial state) of L = Σ dy·y + Σ dh·h_final against
    central differences of the forward oracle, on a small gated problem."""
    rng = _rng(31)
    b, d, L, N = 2, 3, 9, 4
    inp = {"x": rng.normal(size=(b, d, L)), "delta": rng.uniform(0.05, 1.2, size=(b, d, L)),
           "A": -rng.uniform(0.2, 2.5, size=(d, N)), "B": rng.normal(size=(b, L, N)),
           "C": rng.normal(size=(b, L, N)), "D": rng.normal(size=d), "z": rng.normal(size=(b, d, L)),
           "h0": rng.normal(size=(b, d, N)) * 0.5}
    dy = rng.normal(size=(b, d, L))
    dhf = rng.normal(size=(b, d, N))
    _fd_check(orc, inp, dy, dhf, ["x", "delta", "A", "B", "C", "D", "z", "h0"])


def pin_bwd_small_and_zero_A(orc):
    """The A derivative where A = 0 (the ZOH limit, ∂β/∂a → Δ²/2) and where |Δ·A| is tiny (the
    series branch), against central differences; no gate."""
    rng = _rng(37)
    b, d, L, N = 1, 2, 7, 4
    A = -rng.uniform(0.2, 2.0, size=(d, N))
    A[0, 1] = 0.0
    A[1, 2] = -3e-4
    A[1, 0] = 2e-3
    inp = {"x": rng.normal(size=(b, d, L)), "delta": rng.uniform(0.1, 1.5, size=(b, d, L)), "A": A,
           "B": rng.normal(size=(b, L, N)), "C": rng.normal(size=(b, L, N)), "D": rng.normal(size=d)}
    dy = rng.normal(size=(b, d, L))
    dhf = np.zeros((b, d, N))
    _fd_check(orc, inp, dy, dhf, ["A", "delta", "x"], rtol=5e-6, atol=1e-8)


def pin_bwd_impulse_closed_form(orc):
    """Scalar LTI impulse (x = δ_0, B = C = 1, D = 0, constant Δ): y_T = β Ā^T, so
    ∂y_T/∂x_0 = β Ā^T, ∂y_T/∂a = β'(a) Ā^T + β T Δ Ā^T, ∂y_T/∂Δ_0 = Ā·Ā^T, ∂y_T/∂Δ_t = β a Ā^T (t ≥ 1)."""
    a, dl, T, L = -0.7, 0.4, 5, 8
    x = np.zeros((1, 1, L)); x[0, 0, 0] = 1.0
    delta = np.full((1, 1, L), dl)
    A = np.array([[a]]); B = np.ones((1, L, 1)); C = np.ones((1, L, 1))
    dy = np.zeros((1, 1, L)); dy[0, 0, T] = 1.0
    g = orc.scan_bwd(x, delta, A, B, C, dy=dy)
    ab = math.exp(dl * a)
    beta = math.expm1(dl * a) / a
    dbeta = (dl * ab - beta) / a
    _close(g["dx"][0, 0, 0], beta * ab ** T, what="dx_0")
    _close(g["dA"][0, 0], dbeta * ab ** T + beta * T * dl * ab ** T, what="dA")
    _close(g["ddelta"][0, 0, 0], ab * ab ** T, what="dΔ_0")
    for t in range(1, T + 1):
        _close(g["ddelta"][0, 0, t], beta * a * ab ** T, what=f"dΔ_{t}")
    for t in range(T + 1, L):
        _close(g["ddelta"][0, 0, t], 0.0, what=f"dΔ_{t} after the observed step")


# ---------------------------------------------------------------------------------------------
# The causal depthwise Conv1D + SiLU front end
# ---------------------------------------------------------------------------------------------
def pin_conv_identity_and_shift(orc):
    """Taps (0, …, 0, 1) and no bias pass the input through (then silu); taps (0, …, 1, 0) delay it
    by one step; a bias alone gives silu(bias) everywhere."""
    rng = _rng(41)
    b, d, L, W = 2, 3, 11, 4
    xin = rng.normal(size=(b, d, L))
    w = np.zeros((d, W)); w[:, -1] = 1.0
    x, _ = orc.conv1d(xin, w, silu=False)
    _close(x, xin, what="identity taps")
    x, _ = orc.conv1d(xin, w, silu=True)
    _close(x, silu_lib(xin), what="identity taps + silu")
    w = np.zeros((d, W)); w[:, -2] = 1.0
    x, _ = orc.conv1d(xin, w, silu=False)
    _close(x[:, :, 1:], xin[:, :, :-1], what="one-step delay")
    _close(x[:, :, 0], np.zeros((b, d)), what="nothing before the sequence")
    bias = rng.normal(size=d)
    x, _ = orc.conv1d(np.zeros((b, d, L)), np.zeros((d, W)), bias=bias)
    _close(x, np.broadcast_to(silu_lib(bias)[None, :, None], (b, d, L)), what="bias only")


def pin_conv_impulse_and_causality(orc):
    """An impulse at t0 reads the taps back in reverse order (u_{t0+j} = w[W-1-j]); changing an input
    never changes an earlier output (the convolution is causal)."""
    rng = _rng(43)
    d, L, W = 2, 12, 4
    w = rng.normal(size=(d, W))
    xin = np.zeros((1, d, L)); xin[0, :, 5] = 1.0
    x, _ = orc.conv1d(xin, w, silu=False)
    for j in range(W):
        _close(x[0, :, 5 + j], w[:, W - 1 - j], what=f"impulse response lag {j}")
    _close(x[0, :, :5], np.zeros((d, 5)), what="before the impulse")
    _close(x[0, :, 5 + W:], np.zeros((d, L - 5 - W)), what="after the window")
    xin = rng.normal(size=(1, d, L))
    xin2 = xin.copy(); xin2[0, :, 7] += 3.0
    x2, _ = orc.conv1d(xin2, w, bias=None)
    x1b, _ = orc.conv1d(xin, w, bias=None)
    _close(x2[:, :, :7], x1b[:, :, :7], what="causality")


def pin_conv_state_chaining(orc):
    """Decode keeps the last W-1 inputs: running the sequence in two calls, the second starting from
    the first call's state, equals one call (kasblo page, section training、prefill、decode)."""
    rng = _rng(47)
    b, d, L, W = 2, 3, 10, 4
    xin = rng.normal(size=(b, d, L)); w = rng.normal(size=(d, W)); bias = rng.normal(size=d)
    st0 = rng.normal(size=(b, d, W - 1))
    x, st = orc.conv1d(xin, w, bias, st0)
    for cut in (1, 2, 6):
        xa, sa = orc.conv1d(xin[:, :, :cut], w, bias, st0)
        xb, sb = orc.conv1d(xin[:, :, cut:], w, bias, sa)
        _close(np.concatenate([xa, xb], axis=2), x, what=f"chained at {cut}")
        _close(sb, st, what=f"state chained at {cut}")
    _close(st, xin[:, :, L - (W - 1):], what="state = last W-1 inputs")


def pin_lti_kernel_scalar_example(orc):
    """kasblo page, scalar example, read as a time-invariant kernel: K̄ for A = -1, Δ = 0.5, B = C = 1
    starts with the four printed weights, and equals (1 - e^{-1/2}) e^{-k/2} (the page's closed forms)."""
    g = _golden_pairs("kasblo_scalar_example.txt")
    half = 0.5 * 10.0 ** (-g["printed_decimals"])
    L = 12
    K = orc.lti_kernel([g["delta"]], [[g["A"]]], [[g["B"]]], [[g["C"]]], L)
    for k in range(4):
        assert abs(K[0, k] - g[f"weight_lag{k}"]) <= half, (k, K[0, k])
    _close(K[0], (1.0 - math.exp(-0.5)) * np.exp(-0.5 * np.arange(L)), what="scalar K closed form")


def pin_lti_kernel_van_loan(orc):
    """K̄_k = C Ā^k B̄ ("State Space Models（SSM）とMamba" §2.3) with Ā, B̄ from the block matrix
    exponential (Van Loan) and Ā^k from a matrix power, per channel; one A entry is 0 (the ZOH limit)."""
    rng = _rng(53)
    d, N, L = 3, 5, 40
    A = -rng.uniform(0.1, 2.5, size=(d, N)); A[1, 3] = 0.0
    dl = rng.uniform(0.02, 0.9, size=d)
    B = rng.normal(size=(d, N)); C = rng.normal(size=(d, N))
    K = orc.lti_kernel(dl, A, B, C, L)
    want = np.empty((d, L))
    for idd in range(d):
        Ab, Bb = zoh_vanloan(A[idd], B[idd], dl[idd])
        want[idd] = [C[idd] @ np.linalg.matrix_power(Ab, k) @ Bb for k in range(L)]
    _close(K, want, rtol=1e-10, atol=1e-12, what="LTI kernel")


def pin_lti_conv_equals_recurrence(orc):
    """The two faces of a fixed SSM (kasblo page, section 固定SSMには「再帰」と「畳み込み」の二つの顔がある):
    the kernel route (K̄, then x ∗ K̄ + D x, gate) equals the recurrent scan run with the same Δ, B, C
    at every step, channel by channel."""
    rng = _rng(59)
    b, d, N, L = 2, 3, 4, 30
    A = -rng.uniform(0.1, 2.0, size=(d, N)); A[2, 1] = 0.0
    dl = rng.uniform(0.05, 1.0, size=d)
    B = rng.normal(size=(d, N)); C = rng.normal(size=(d, N)); D = rng.normal(size=d)
    x = rng.normal(size=(b, d, L)); z = rng.normal(size=(b, d, L))
    y = orc.lti_conv(x, orc.lti_kernel(dl, A, B, C, L), D=D, z=z)
    for idd in range(d):
        yr, _ = orc.scan_fwd(x[:, idd:idd + 1], np.full((b, 1, L), dl[idd]), A[idd:idd + 1],
                             np.broadcast_to(B[idd], (b, L, N)), np.broadcast_to(C[idd], (b, L, N)),
                             D=D[idd:idd + 1], z=z[:, idd:idd + 1])
        _close(y[:, idd:idd + 1], yr, rtol=1e-10, atol=1e-12, what=f"LTI conv vs recurrence, channel {idd}")


def pin_lti_conv_library(orc):
    """y = x ∗ K̄ + D x (then silu(z)) against numpy's full convolution truncated to L, for arbitrary K̄."""
    rng = _rng(61)
    b, d, L = 2, 3, 25
    x = rng.normal(size=(b, d, L)); K = rng.normal(size=(d, L)); D = rng.normal(size=d)
    z = rng.normal(size=(b, d, L))
    want = np.empty((b, d, L))
    for ib in range(b):
        for idd in range(d):
            want[ib, idd] = np.convolve(x[ib, idd], K[idd])[:L] + D[idd] * x[ib, idd]
    _close(orc.lti_conv(x, K, D=D), want, what="LTI conv, no gate")
    _close(orc.lti_conv(x, K, D=D, z=z), want * silu_lib(z), what="LTI conv, gated")
    _close(orc.lti_conv(x, K), want - D[None, :, None] * x, what="LTI conv, no D")


def pin_ssd_duality(orc):
    """Scalar decay per head: the quadratic (masked-attention) form equals the recurrent scan run with
    Δ repeated over the head's channels and A = a_h on every state (the recurrence unrolled; pages:
    Mamba-2's state space duality of SSMs and linear attention). One head has a = 0."""
    rng = _rng(67)
    b, H, P, L, N = 2, 3, 2, 11, 4
    x = rng.normal(size=(b, H * P, L)); z = rng.normal(size=(b, H * P, L))
    dl = rng.uniform(0.05, 1.0, size=(b, H, L))
    A = -rng.uniform(0.2, 2.0, size=H); A[1] = 0.0
    B = rng.normal(size=(b, L, N)); C = rng.normal(size=(b, L, N)); D = rng.normal(size=H * P)
    y = orc.ssd_quadratic(x, dl, A, B, C, D=D, z=z)
    yr, _ = orc.scan_fwd(x, np.repeat(dl, P, axis=1), np.repeat(A, P)[:, None].repeat(N, axis=1), B, C, D=D, z=z)
    _close(y, yr, rtol=1e-10, atol=1e-12, what="SSD quadratic form vs recurrence")


def pin_ssd_masked_attention(orc):
    """With A = 0 and Δ = 1 the form is plain causal linear attention, y = tril(C Bᵀ) x (queries C, keys B,
    values x); with a constant Δ and a ≠ 0 the mask is the Toeplitz decay exp(aΔ(t−s)) and the values
    carry β = (e^{aΔ} − 1)/a. Both built with numpy matrix products."""
    rng = _rng(71)
    b, H, P, L, N = 1, 2, 3, 10, 5
    x = rng.normal(size=(b, H * P, L)); B = rng.normal(size=(b, L, N)); C = rng.normal(size=(b, L, N))
    G = np.tril(C[0] @ B[0].T)
    y = orc.ssd_quadratic(x, np.ones((b, H, L)), np.zeros(H), B, C)
    _close(y[0], x[0] @ G.T, what="linear attention")
    a, dlt = np.array([-0.6, -1.7]), 0.3
    y = orc.ssd_quadratic(x, np.full((b, H, L), dlt), a, B, C)
    t = np.arange(L)
    for h in range(H):
        mask = np.tril(np.exp(a[h] * dlt * (t[:, None] - t[None, :])))
        beta = np.expm1(a[h] * dlt) / a[h]
        want = (x[0, h * P:(h + 1) * P] * beta) @ (G * mask).T
        _close(y[0, h * P:(h + 1) * P], want, what=f"decayed attention, head {h}")


def pin_softplus_closed_forms(orc):
    """softplus(v) = log(1 + e^v): ln 2 at 0; softplus(v) − softplus(−v) = v; the inverse of
    c ↦ log(e^c − 1); e^v to full relative precision far below 0; v far above 0."""
    import oracle as O
    _close(O.softplus(0.0), math.log(2.0), rtol=1e-15, what="softplus(0)")
    v = _rng(41).normal(0.0, 5.0, size=200)
    _close(O.softplus(v) - O.softplus(-v), v, rtol=1e-13, atol=1e-13, what="softplus odd part")
    c = np.array([1e-6, 0.01, 0.5, 3.0, 20.0])
    _close(O.softplus(np.log(np.expm1(c))), c, rtol=1e-12, what="softplus inverse")
    _close(O.softplus(-40.0), math.exp(-40.0), rtol=1e-12, atol=0.0, what="softplus far left")
    _close(O.softplus(800.0), 800.0, rtol=1e-15, what="softplus far right")
    assert np.all(O.softplus(v) > np.maximum(v, 0.0)), "softplus exceeds max(v, 0)"


def pin_fused_front_end_composition(orc):
    """The Conv1D + SiLU → Δ preprocessing → scan composition: with one unit tap and no biases it is the
    scan of silu(xin) (library expit) on the raw Δ; its Conv1D state output is the last W − 1 inputs;
    two calls chained through both states equal one call; L decode steps equal the prefill."""
    rng = _rng(43)
    b, d, L, N, W = 2, 5, 30, 4, 4
    xin = rng.standard_normal((b, d, L))
    dl = rng.normal(-1.0, 0.7, size=(b, d, L))
    A = -rng.uniform(0.2, 2.0, size=(d, N))
    B, C = rng.standard_normal((b, L, N)), rng.standard_normal((b, L, N))
    D, z = rng.standard_normal(d), rng.standard_normal((b, d, L))
    # one unit tap, no bias, no softplus: the plain scan of silu(xin)
    y1, h1, _, x1 = orc.scan_fwd_conv(xin, np.ones((d, 1)), None, None, np.abs(dl), None, False, A, B, C, D, z)
    y2, h2 = orc.scan_fwd(silu_lib(xin), np.abs(dl), A, B, C, D, z)
    _close(y1, y2, what="fused, W = 1: y")
    _close(h1, h2, what="fused, W = 1: state")
    _close(x1, silu_lib(xin), what="fused, W = 1: x")
    # W = 4 with biases and softplus: the state output and chaining
    w = rng.normal(0.0, 0.5, size=(d, W))
    cb, db = rng.standard_normal(d), rng.normal(0.0, 0.3, size=d)
    cs0 = rng.standard_normal((b, d, W - 1))
    h0 = rng.standard_normal((b, d, N)) * 0.3
    y, h, cs, _ = orc.scan_fwd_conv(xin, w, cb, cs0, dl, db, True, A, B, C, D, z, h0)
    assert np.array_equal(cs, xin[:, :, L - (W - 1):]), "Conv1D state output is not the last W - 1 inputs"
    cut = 11
    ya, ha, csa, _ = orc.scan_fwd_conv(xin[:, :, :cut], w, cb, cs0, dl[:, :, :cut], db, True, A, B[:, :cut],
                                       C[:, :cut], D, z[:, :, :cut], h0)
    yb, hb, csb, _ = orc.scan_fwd_conv(xin[:, :, cut:], w, cb, csa, dl[:, :, cut:], db, True, A, B[:, cut:],
                                       C[:, cut:], D, z[:, :, cut:], ha)
    _close(np.concatenate([ya, yb], axis=2), y, what="fused chained y")
    _close(hb, h, what="fused chained state")
    _close(csb, cs, what="fused chained Conv1D state")
    # decode steps
    st, cst = h0.copy(), cs0.copy()
    ys = []
    for t in range(L):
        yt, st, cst, _ = orc.scan_step_conv(st, cst, xin[:, :, t], w, cb, dl[:, :, t], db, True, A, B[:, t], C[:, t],
                                            D, z[:, :, t])
        ys.append(yt)
    _close(np.stack(ys, axis=2), y, what="fused decode steps vs prefill")
    _close(st, h, what="fused decode state")
    _close(cst, cs, what="fused decode Conv1D state")


ALL_PINS = [
    pin_scalar_worked_example,
    pin_delta_gate,
    pin_decay_impulse,
    pin_cumulative_sum,
    pin_lti_convolution,
    pin_selective_unroll,
    pin_closed_gate,
    pin_delta_limits,
    pin_affine_associativity,
    pin_prefill_equals_decode,
    pin_skip_and_gate,
    pin_linearity,
    pin_bwd_finite_differences,
    pin_bwd_small_and_zero_A,
    pin_bwd_impulse_closed_form,
    pin_conv_identity_and_shift,
    pin_conv_impulse_and_causality,
    pin_conv_state_chaining,
    pin_lti_kernel_scalar_example,
    pin_lti_kernel_van_loan,
    pin_lti_conv_equals_recurrence,
    pin_lti_conv_library,
    pin_ssd_duality,
    pin_ssd_masked_attention,
    pin_softplus_closed_forms,
    pin_fused_front_end_composition,
]
