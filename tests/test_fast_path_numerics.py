"""fp32 emulation of the prefill kernel's per-step arithmetic, checked against the fp64 oracle (no GPU).

The fast prefill path keeps the scaled state s = A·h and takes the zero-order-hold input from
Ā − 1 (page "Mambaとは？Transformer以外の系列モデル", section 状態空間モデルを一つの式から理解する:
B̄ = (ΔA)⁻¹(exp(ΔA) − I)ΔB), with Ā = 2^(Δ·A·log2 e) from the hardware exp. Ā is a float32 near 1,
so Ā − 1 carries an absolute error of about 2⁻²⁴ whatever |Δ·A| is: a relative error of about
6e-8/|Δ·A| in B̄. Where Δ·A stays small for many steps (a slow channel), that exceeds the fp32 bar.

The kernel therefore classifies each tile of steps, per wavefront: when some valid state of some
channel has a mean |Δ·A·log2 e| over the tile below a threshold, the wavefront runs that tile with the
coefficient taken per step from the cubic series of 2^u − 1 wherever |u| < 1/16 (the accurate tile);
other tiles keep Ā − 1. In a kept tile the per-step errors add up in quadrature against increments
whose mean size is at least the threshold, so the state's relative error stays near 2⁻²⁴ divided by
that threshold.

This module emulates those operations in float32 (fused multiply-adds rounded once) with three models
of the hardware exp2: correctly rounded, a random error of up to one unit in the last place, and a
one-sided error of one unit. It shows the raw coefficient failing the fp32 bar in the slow regime and
the classified rule passing it everywhere tested; it also measures how often the rule fires on the
workloads' own distributions (each accurate tile costs about half again the VALU work of a kept one).
The emulation is a model of the kernel written for this test; the oracle is the reference.
"""
import numpy as np
import pytest

import oracle
from selective_state_space_82_amd import inputs as I

F32 = np.float32
LOG2E = F32(1.4426950408889634)
LN2 = 0.6931471805599453
# cubic series of 2^u - 1 = u·(c1 + u·(c2 + u·c3)), and where the kernel uses it
C1, C2, C3 = F32(LN2), F32(LN2 ** 2 / 2), F32(LN2 ** 3 / 6)
POLY_U = F32(1.0 / 16.0)
# mean |u| over a tile below which the tile runs accurate, per storage type (u = Δ·A·log2 e)
CLASS_MEAN_U = {"f32": F32(2.0 ** -7), "bf16": F32(2.0 ** -12)}
K_TILE = {"f32": 16, "bf16": 32}
TAU = {"f32": 1e-4, "bf16": 2e-2}


def fma(a, b, c):
    """float32 fused multiply-add (the product is exact in float64; one final rounding)."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F32)


def make_exp2(model, seed=0):
    rng = np.random.default_rng(seed)

    def exp2(u):
        r = np.exp2(u.astype(np.float64)).astype(F32)
        if model == "rn":
            return r
        if model == "ulp":      # up to one unit in the last place, either way
            step = rng.integers(-1, 2, size=r.shape)
        elif model == "down":   # one unit toward zero, every time
            step = -np.ones(r.shape, dtype=np.int64)
        else:
            raise ValueError(model)
        up, dn = np.nextafter(r, F32(np.inf)), np.nextafter(r, F32(0.0))
        return np.where(step > 0, up, np.where(step < 0, dn, r)).astype(F32)

    return exp2


def emulate_prefill(inp, rule, exp_model="rn", G=4, npl=4, wave_channels=16):
    """The fast path's arithmetic on fp32 or bf16 inputs (widened), one wavefront per 16 channels of a
    batch row. rule: "raw" (Ā − 1 always), "classified" (the kernel's rule). Returns (y, h, fraction of
    wavefront tiles that ran accurate)."""
    dt = inp["dtype"]
    w = lambda k: None if inp[k] is None else I.widen(inp[k], dt).astype(F32)
    x, dl, z, B, C = w("x"), w("delta"), w("z"), w("B"), w("C")
    A = inp["A"].astype(F32)
    D = np.zeros(A.shape[0], F32) if inp["D"] is None else inp["D"].astype(F32)
    b, d, L = x.shape
    N = A.shape[1]
    assert N == G * npl and d % wave_channels == 0
    exp2 = make_exp2(exp_model)
    a2 = (A * LOG2E).astype(F32)
    ia = (F32(1.0) / A).astype(F32)
    s = np.zeros((b, d, N), F32)
    y = np.empty((b, d, L), F32)
    kt = K_TILE[dt]
    thr = (F32(kt) * CLASS_MEAN_U[dt] / np.abs(a2).min(axis=1)).astype(F32)  # per channel
    accurate_tiles = total_tiles = 0
    for t0 in range(0, L, kt):
        t1 = min(L, t0 + kt)
        if rule == "classified":
            dsum = dl[:, :, t0:t1].sum(axis=2, dtype=F32)
            need = (dsum < thr[None, :]).reshape(b, d // wave_channels, wave_channels).any(axis=2)
            acc_tile = np.repeat(need, wave_channels, axis=1)[:, :, None]
            accurate_tiles += int(need.sum())
        total_tiles += b * (d // wave_channels)
        for t in range(t0, t1):
            xt = x[:, :, t][:, :, None]
            u = (dl[:, :, t][:, :, None] * a2[None]).astype(F32)
            em1 = (exp2(u) - F32(1.0)).astype(F32)
            if rule == "classified":
                p = fma(u, C3, C2)
                p = fma(u, p, C1)
                em1p = (u * p).astype(F32)
                em1 = np.where(acc_tile & (np.abs(u) < POLY_U), em1p, em1).astype(F32)
            pre = fma(B[:, t][:, None, :], xt, s)
            s = fma(em1, pre, s)
            cia = (C[:, t][:, None, :] * ia[None]).astype(F32)
            part = np.zeros((b, d, G), F32)
            for j in range(npl):
                idx = np.arange(G) * npl + j
                part = fma(cia[:, :, idx], s[:, :, idx], part)
            v = part[:, :, 0]
            for g in range(1, G):
                v = (v + part[:, :, g]).astype(F32)
            yt = fma(D[None, :], x[:, :, t], v)
            if z is not None:
                zt = z[:, :, t]
                sig = (F32(1.0) / (F32(1.0) + exp2((-LOG2E * zt).astype(F32)))).astype(F32)
                yt = (yt * (zt * sig).astype(F32)).astype(F32)
            y[:, :, t] = yt
    h = (s * ia[None]).astype(F32)
    frac = accurate_tiles / total_tiles if rule == "classified" else 0.0
    return y, h, frac


def rel_err(got, ref):
    return float(np.max(np.abs(got.astype(np.float64) - ref) / (1.0 + np.abs(ref))))


def oracle_ref(inp):
    dt = inp["dtype"]
    w = lambda k: None if inp[k] is None else I.widen(inp[k], dt)
    return oracle.scan_fwd(w("x"), w("delta"), inp["A"], w("B"), w("C"), inp["D"], w("z"))


# The slow regime: Δ·A small for many steps in a row (channels whose decay is slow).
SLOW_CASES = {
    "A=-0.01,delta=0.01": dict(L=2048, a_value=-0.01, delta_value=0.01),
    "A=-0.002,delta=0.005": dict(L=4096, a_value=-0.002, delta_value=0.005),
    "A~-U(2^-10,0.05),delta=softplus(N(-5,1))": dict(L=2048, a_kind="small", delta_mu=-5.0),
}
# The workloads' own distributions at a reduced size (fp32 storage, the strict bar).
WORKLOAD_CASES = {
    "130M-like": dict(L=2048, a_kind="neg_index", delta_mu=-3.0, delta_sigma=1.0),
    "1.4B-like": dict(L=2048, a_kind="neg_index", delta_mu=-2.0, delta_sigma=0.5),
    "long-context-like": dict(L=4096, a_kind="neg_index_u", delta_mu=-4.0, delta_sigma=1.0),
}


def case_inputs(kw, dtype="f32", d=32, seed=3):
    kw = dict(kw)
    L = kw.pop("L")
    return I.random_prefill(1, d, L, 16, dtype=dtype, seed=seed, **kw)


@pytest.mark.parametrize("name", list(SLOW_CASES))
def test_raw_coefficient_fails_fp32_bar_in_slow_regime(name):
    """Ā − 1 from a float32 Ā, even correctly rounded, breaks the 1e-4 bar where Δ·A stays small."""
    inp = case_inputs(SLOW_CASES[name])
    yr, hr = oracle_ref(inp)
    y, h, _ = emulate_prefill(inp, "raw", "rn")
    err = max(rel_err(y, yr), rel_err(h, hr))
    print(f"[raw {name}] max rel err {err:.2e}")
    assert err > TAU["f32"], err


@pytest.mark.parametrize("model", ["rn", "ulp", "down"])
@pytest.mark.parametrize("name", list(SLOW_CASES) + list(WORKLOAD_CASES))
def test_classified_rule_meets_fp32_bar(name, model):
    """With the per-tile classification every case stays a factor 4 inside the fp32 bar, whichever
    exp2 error model holds."""
    kw = SLOW_CASES.get(name) or WORKLOAD_CASES[name]
    inp = case_inputs(kw)
    yr, hr = oracle_ref(inp)
    y, h, frac = emulate_prefill(inp, "classified", model)
    ey, eh = rel_err(y, yr), rel_err(h, hr)
    print(f"[classified {name} exp2={model}] y {ey:.2e} h {eh:.2e}, accurate tiles {frac:.3f}")
    assert ey <= TAU["f32"] / 4 and eh <= TAU["f32"] / 4, (ey, eh)
    if name in SLOW_CASES:
        assert frac > 0.9  # the slow regime runs accurate


@pytest.mark.parametrize("name", list(SLOW_CASES))
def test_classified_rule_meets_bf16_bar(name):
    inp = case_inputs(SLOW_CASES[name], dtype="bf16")
    yr, hr = oracle_ref(inp)
    y, h, _ = emulate_prefill(inp, "classified", "ulp")
    # the emulation keeps y in fp32; the kernel's bf16 rounding of y adds at most 2^-9 relative
    assert rel_err(y, yr) <= TAU["bf16"] / 8 and rel_err(h, hr) <= TAU["bf16"] / 8


def accurate_tile_rate(kw, dtype, d=256, L=4096, seed=11):
    """Fraction of wavefront tiles the classification sends to the accurate variant (no scan needed:
    it depends on Δ and A only)."""
    kw = dict(kw)
    kw.pop("L", None)
    inp = I.random_prefill(1, d, L, 16, dtype=dtype, seed=seed, gate=False, **kw)
    dl = I.widen(inp["delta"], dtype).astype(F32)[0]
    a2 = (inp["A"].astype(F32) * LOG2E).astype(F32)
    kt = K_TILE[dtype]
    thr = (F32(kt) * CLASS_MEAN_U[dtype] / np.abs(a2).min(axis=1)).astype(F32)
    sums = dl[:, : (L // kt) * kt].reshape(d, L // kt, kt).sum(axis=2, dtype=F32)
    need = (sums < thr[:, None]).reshape(d // 16, 16, L // kt).any(axis=1)
    return float(need.mean())


@pytest.mark.parametrize("name,dtype,limit", [("130M-like", "f32", 0.01), ("1.4B-like", "bf16", 0.001),
                                              ("long-context-like", "bf16", 0.01)])
def test_classification_rarely_fires_on_workload_distributions(name, dtype, limit):
    rate = accurate_tile_rate(WORKLOAD_CASES[name], dtype)
    print(f"[{name} {dtype}] accurate tiles {rate:.4f}")
    assert rate <= limit, rate
