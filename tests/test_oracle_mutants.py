"""Plausible mistakes planted in a copy of the oracle source must each fail at least one pin.

The mutants are compiled from text substitutions on the CPU only; the real oracle is untouched.
"""
import os

import numpy as np
import pytest

import oracle
from pins import ALL_PINS

MUTANTS = {
    "drop_skip_D": ("double yt = acc + dskip * xt;", "double yt = acc;"),
    "exp_sign": ("*abar = exp(u);", "*abar = exp(-u);"),
    "euler_bbar": ("expm1(u) / a", "u / a"),
    "a0_limit_zero": (": delta;", ": 0.0;"),
    "no_decay": ("h[n] = abar * h[n] +", "h[n] = h[n] +"),
    "readout_before_update": (
        "            h[n] = abar * h[n] + bcoef * Bt[t * N + n] * xt;\n"
        "            /* y_t = C h_t with the just-updated state (both pages update first, then read). */\n"
        "            acc += Ct[t * N + n] * h[n];",
        "            acc += Ct[t * N + n] * h[n];\n"
        "            h[n] = abar * h[n] + bcoef * Bt[t * N + n] * xt;"),
    "B_transposed": ("bcoef * Bt[t * N + n]", "bcoef * Bt[n * L + t]"),
    "C_transposed": ("acc += Ct[t * N + n]", "acc += Ct[n * L + t]"),
    "sigmoid_gate": ("return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    "A_channel0": ("delta + row * (size_t)L, A + (size_t)id * (size_t)N,", "delta + row * (size_t)L, A,"),
    "step_A_channel0": ("scan_row(x + row, delta + row, A + (size_t)id * (size_t)N,",
                        "scan_row(x + row, delta + row, A,"),
    "step_B_batch0": ("B + (size_t)ib * (size_t)N,\n                     C + (size_t)ib * (size_t)N,",
                      "B,\n                     C + (size_t)ib * (size_t)N,"),
    "B_batch0": ("B + (size_t)ib * (size_t)L * (size_t)N, C", "B, C"),
    "ignore_h0": ("hrow[n] = h0 ? h0[row * (size_t)N + (size_t)n] : 0.0;", "hrow[n] = 0.0;"),
    "gate_on_skip_only": ("if (z) yt *= silu(z[t]);", "if (z) yt = acc + dskip * xt * silu(z[t]);"),
    # gradients
    "bwd_state_after_step": ("const double dab = ln * hp[n];", "const double dab = ln * h[n];"),
    "bwd_no_adjoint_decay": ("lam[n] = abar * ln;", "lam[n] = ln;"),
    "bwd_dbeta_da_sign": ("return (delta * abar - beta) / a;", "return (delta * abar + beta) / a;"),
    "bwd_series_coefficient": ("term = (double)(k + 1) * vk / fact;", "term = vk / fact;"),
    "bwd_silu_derivative": ("(1.0 + zr[t] * (1.0 - sg))", "(1.0 + zr[t] * sg)"),
    "bwd_ddelta_drops_beta": ("gd += dab * a[n] * abar + dbe * abar;", "gd += dab * a[n] * abar;"),
    "bwd_dB_drops_x": ("+= ln * beta * xt;", "+= ln * beta;"),
    "bwd_dD_ungated": ("if (dD) dD[id] += dys * xt;", "if (dD) dD[id] += dyr[t] * xt;"),
    "bwd_dC_old_state": ("+= dys * h[n];", "+= dys * hp[n];"),
    "bwd_dh0_undecayed": ("dh0[row * (size_t)N + (size_t)n] = lam[n];", "dh0[row * (size_t)N + (size_t)n] = lam[n] * 0.5;"),
    # causal conv1d
    "conv_taps_reversed": ("u += w[(size_t)id * (size_t)W + (size_t)k] * ext[t + k];",
                           "u += w[(size_t)id * (size_t)W + (size_t)(W - 1 - k)] * ext[t + k];"),
    "conv_off_by_one": ("u += w[(size_t)id * (size_t)W + (size_t)k] * ext[t + k];",
                        "u += w[(size_t)id * (size_t)W + (size_t)k] * ext[t + k + (t + k + 1 < L + H ? 1 : 0)];"),
    "conv_state_ignored": ("ext[k] = state_in ? state_in[row * (size_t)H + (size_t)k] : 0.0;", "ext[k] = 0.0;"),
    "conv_state_first_inputs": ("state_out[row * (size_t)H + (size_t)k] = ext[L + k];",
                                "state_out[row * (size_t)H + (size_t)k] = ext[H + k];"),
    "conv_bias_dropped": ("double u = bias ? bias[id] : 0.0;", "double u = 0.0;"),
    "lti_power_from_abar": ("double power = 1.0; /* Ā^k */", "double power = abar; /* Ā^k */"),
    "lti_euler_bbar": ("const double cb = C[i] * bcoef * B[i];", "const double cb = C[i] * delta[id] * B[i];"),
    "lti_channel0_params": ("const size_t i = (size_t)id * (size_t)N + (size_t)n;", "const size_t i = (size_t)n;"),
    "lti_kernel_index": ("acc += Kd[t - s] * x[row + (size_t)s];", "acc += Kd[s] * x[row + (size_t)s];"),
    "lti_drop_D": ("double yt = acc + (D ? D[id] : 0.0) * x[row + (size_t)t];", "double yt = acc;"),
    "lti_gate_dropped": ("if (z) yt *= silu(z[row + (size_t)t]);\n                y[row + (size_t)t] = yt;",
                         "y[row + (size_t)t] = yt;"),
    "ssd_strict_mask": ("for (long s = 0; s <= t; ++s) {", "for (long s = 0; s < t; ++s) {"),
    "ssd_decay_from_s": ("for (long r = s + 1; r <= t; ++r) sum += dl[r];", "for (long r = s; r <= t; ++r) sum += dl[r];"),
    "ssd_beta_dropped": ("acc += cb * exp(a * sum) * beta_s * xr[s];", "acc += cb * exp(a * sum) * xr[s];"),
    "ssd_beta_at_t": ("oracle_zoh(dl[s], a, &abar_s, &beta_s);", "oracle_zoh(dl[t], a, &abar_s, &beta_s);"),
    "ssd_key_at_t": ("cb += Cb[(size_t)t * (size_t)N + (size_t)n] * Bb[(size_t)s * (size_t)N + (size_t)n];",
                     "cb += Cb[(size_t)t * (size_t)N + (size_t)n] * Bb[(size_t)t * (size_t)N + (size_t)n];"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE, encoding="utf-8") as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new), encoding="utf-8")
    lib = oracle.compile_library(str(src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(orc)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
