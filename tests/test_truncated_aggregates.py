"""The reading behind the truncated aggregate walk, checked with the fp64 oracle (no GPU).

A segment's end state from zero splits at any step t_s into the part from the steps after t_s and the decayed
state there (page "Mambaとは？Transformer以外の系列モデル", section Selective Scanは選択機構そのものではない: the
per-step affine maps compose associatively):
    E[0, T) = E[t_s, T) + R·h(t_s),   R = Π_{u >= t_s} Ā_u = exp(A·Σ_{u >= t_s} Δ_u),
where h(t_s) is the state from zero just before t_s. The aggregate pass stops its backward walk at the first
tile boundary t_s where R <= 2^-24 (fp32's unit roundoff) for every state of a wavefront, so the part it
drops is R·h(t_s), at most 2^-24·|h(t_s)|: no more than the error of holding h(t_s) in fp32. These tests
check the identity and that bound on Mamba-shaped inputs (including Δ < 0 steps and the long-context decay
rates), and that the walk's stopping rule on ΣΔ gives R <= 2^-24.
"""
import numpy as np
import pytest

import oracle
from selective_state_space_82_amd import inputs as I


def _end_state(x, delta, A, B, h0=None):
    """The oracle's final state [d, N] of one batch row over the given steps (C, D, z do not enter it)."""
    d, T = x.shape
    C = np.zeros_like(B)
    _, h = oracle.scan_fwd(x[None], delta[None], A, B[None], C[None], None, None, None if h0 is None else h0[None])
    return h[0]


@pytest.mark.parametrize("case", [
    dict(delta_mu=-4.0, a_kind="neg_index_u", T=2048),  # the long-context recipe's decay rates
    dict(delta_mu=-2.0, a_kind="neg_index", T=1024),
    dict(delta_mu=0.0, a_kind="random", T=512),
])
def test_split_identity_and_stop_bound(case):
    d, N, T = 16, 16, case["T"]
    inp = I.random_prefill(1, d, T, N, dtype="f32", seed=T, delta_mu=case["delta_mu"], a_kind=case["a_kind"])
    x = I.widen(inp["x"], "f32")[0].astype(np.float64)
    dl = I.widen(inp["delta"], "f32")[0].astype(np.float64)
    B = I.widen(inp["B"], "f32")[0].astype(np.float64)
    A = inp["A"].astype(np.float64)
    full = _end_state(x, dl, A, B)
    # the backward walk's stopping point, tile by tile (32 steps), per state group of four
    tail = np.cumsum(dl[:, ::-1], axis=1)[:, ::-1]          # Σ_{u >= t} Δ_u per channel
    stopped = 0
    for g in range(N // 4):
        a = A[:, 4 * g:4 * g + 4]                             # [d, 4]
        ts = 0
        for t in range(T - 32, 0, -32):
            R = np.exp(a * tail[:, t][:, None])               # Π_{u >= t} Ā_u per (channel, state)
            if np.all(R <= 2.0 ** -24):
                ts = t
                break
        if ts == 0:
            continue
        stopped += 1
        R = np.exp(a * tail[:, ts][:, None])
        assert np.all(R <= 2.0 ** -24)
        trunc = _end_state(x[:, ts:], dl[:, ts:], A, B[ts:])[:, 4 * g:4 * g + 4]
        h_ts = _end_state(x[:, :ts], dl[:, :ts], A, B[:ts])[:, 4 * g:4 * g + 4]
        # the identity, to fp64 rounding
        np.testing.assert_allclose(full[:, 4 * g:4 * g + 4], trunc + R * h_ts, rtol=1e-12, atol=1e-12)
        # the dropped part against the state at the stop
        assert np.all(np.abs(full[:, 4 * g:4 * g + 4] - trunc) <= 2.0 ** -24 * np.abs(h_ts) + 1e-12)
    assert stopped >= 1, "no state group stops early on these inputs: the case tests nothing"


def test_split_identity_with_negative_delta():
    """Δ < 0 steps before the split change h(t_s) and P, not the identity; P over the whole segment still counts
    them (exp(A·ΣΔ) over all steps)."""
    d, N, T = 8, 16, 600
    inp = I.random_prefill(1, d, T, N, dtype="f32", seed=3, delta_mu=0.0)
    x = I.widen(inp["x"], "f32")[0].astype(np.float64)
    dl = I.widen(inp["delta"], "f32")[0].astype(np.float64)
    dl[:, 40:46] = -0.08
    B = I.widen(inp["B"], "f32")[0].astype(np.float64)
    A = inp["A"].astype(np.float64)
    ts = 320
    full = _end_state(x, dl, A, B)
    R = np.exp(A * dl[:, ts:].sum(axis=1)[:, None])
    trunc = _end_state(x[:, ts:], dl[:, ts:], A, B[ts:])
    h_ts = _end_state(x[:, :ts], dl[:, :ts], A, B[:ts])
    np.testing.assert_allclose(full, trunc + R * h_ts, rtol=1e-10, atol=1e-12)
    # and P = Π Ā over the segment is the carry's multiplier: chaining (P, E) reproduces the state through a
    # following segment
    h1 = _end_state(x, dl, A, B, h0=np.ones((d, N)))
    P = np.exp(A * dl.sum(axis=1)[:, None])
    np.testing.assert_allclose(h1, P * 1.0 + full, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("case", [
    dict(delta_mu=-4.0, a_kind="neg_index_u", T=2944, neg=False),  # the long-context recipe, its segment length
    dict(delta_mu=-2.0, a_kind="neg_index", T=1024, neg=False),
    dict(delta_mu=0.0, a_kind="random", T=600, neg=True),          # Δ < 0 steps before the stop
])
def test_early_stop_drops_the_carried_term_within_a_rounding(case):
    """A walk that stops early (R <= 2^-24 for every state of its group at a tile boundary t_s) leaves P = 0.
    The term it drops from the segment's map, P·h_in, equals R·g(t_s), g(t_s) being the carried-in state h_in
    taken to t_s without inputs (the state from h_in minus the state from zero there): it is at most 2^-24 times
    those states, one fp32 rounding of a state at t_s. Where Δ >= 0 and A <= 0, P <= R <= 2^-24 as well."""
    d, N, T = 16, 16, case["T"]
    inp = I.random_prefill(1, d, T, N, dtype="f32", seed=T + 7, delta_mu=case["delta_mu"], a_kind=case["a_kind"])
    x = I.widen(inp["x"], "f32")[0].astype(np.float64)
    dl = I.widen(inp["delta"], "f32")[0].astype(np.float64)
    if case["neg"]:
        dl[:, 40:46] = -0.08
    B = I.widen(inp["B"], "f32")[0].astype(np.float64)
    A = inp["A"].astype(np.float64)
    h_in = np.random.default_rng(T).standard_normal((d, N)) * 3.0
    tail = np.cumsum(dl[:, ::-1], axis=1)[:, ::-1]
    P = np.exp(A * dl.sum(axis=1)[:, None])
    full_from_h = _end_state(x, dl, A, B, h0=h_in)
    full_from_0 = _end_state(x, dl, A, B)
    np.testing.assert_allclose(full_from_h, P * h_in + full_from_0, rtol=1e-10, atol=1e-12)
    stopped = 0
    for g in range(N // 4):
        a = A[:, 4 * g:4 * g + 4]
        ts = 0
        for t in range(T - 32, 0, -32):
            if np.all(np.exp(a * tail[:, t][:, None]) <= 2.0 ** -24):
                ts = t
                break
        if ts == 0:
            continue
        stopped += 1
        sl = slice(4 * g, 4 * g + 4)
        h_t = _end_state(x[:, :ts], dl[:, :ts], A, B[:ts], h0=h_in)[:, sl]   # the state at t_s from h_in
        h0_t = _end_state(x[:, :ts], dl[:, :ts], A, B[:ts])[:, sl]           # and from zero
        dropped = (P * h_in)[:, sl]
        assert np.all(np.abs(dropped) <= 2.0 ** -24 * (np.abs(h_t) + np.abs(h0_t)) + 1e-12)
        if not case["neg"]:
            assert np.all(P[:, sl] <= 2.0 ** -24)
    assert stopped >= 1, "no state group stops early on these inputs: the case tests nothing"
