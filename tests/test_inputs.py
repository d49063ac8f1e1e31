"""The seeded input generator: determinism, shapes, distributions and bf16 rounding (CPU only)."""
import numpy as np
import pytest
import torch

from selective_state_space_82_amd import inputs as I


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000), rng.standard_normal(1000) * 1e-30,
                        rng.standard_normal(1000) * 1e30, [0.0, -0.0, 1.0, -2.5]]).astype(np.float32)
    ours = I.bf16_bits_from_f64(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_single_rounding_from_f64():
    # values just above a bf16 halfway point that fp32 nearest rounding would pull onto the tie
    base = 1.0 + 2.0 ** -8            # exact halfway between two bf16 neighbours of 1.0
    v = np.array([base + 2.0 ** -40, base - 2.0 ** -40, base])
    got = I.bf16_bits_to_f32(I.bf16_bits_from_f64(v)).astype(np.float64)
    assert got[0] == 1.0 + 2.0 ** -7   # above the tie: up
    assert got[1] == 1.0               # below the tie: down
    assert got[2] == 1.0               # on the tie: to even


def test_widen_is_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        f = I.widen(bits, "bf16")
    finite = np.isfinite(f)
    assert np.array_equal(I.bf16_bits_from_f64(f[finite]), bits[finite])


def test_prefill_deterministic_and_shaped():
    a = I.prefill_inputs("tiny_f32_b1_d8_L128_N4", seed=0)
    b = I.prefill_inputs("tiny_f32_b1_d8_L128_N4", seed=0)
    c = I.prefill_inputs("tiny_f32_b1_d8_L128_N4", seed=1)
    for k in ("x", "delta", "A", "B", "C", "D"):
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], c["x"])
    assert a["z"] is None
    assert a["x"].shape == (1, 8, 128) and a["B"].shape == (1, 128, 4) and a["A"].shape == (8, 4)
    assert np.array_equal(a["A"], -(np.arange(4) + 1.0)[None, :].repeat(8, 0))
    # chunking and threading do not change the draw
    t1 = I.prefill_inputs("tiny_f32_b1_d8_L128_N4", seed=0, threads=1)
    assert np.array_equal(t1["x"], a["x"])


def test_prefill_distributions():
    w = I.WORKLOADS["mamba130m_f32_b4_d1536_L2048_N16"]
    small = I.random_prefill(2, 256, 512, 16, dtype="f32", delta_mu=w.delta_mu, delta_sigma=w.delta_sigma)
    dl = small["delta"].astype(np.float64)
    assert np.all(dl > 0)
    pre = np.log(np.expm1(dl))        # invert softplus
    assert abs(pre.mean() - w.delta_mu) < 0.02 and abs(pre.std() - w.delta_sigma) < 0.02
    x = small["x"].astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_longctx_A_uniform_scaling():
    w = I.WORKLOADS["longctx_bf16_b1_d2048_L131072_N16"]
    A = I._a_matrix(0, w.name, w.d, w.N, w.a_kind).astype(np.float64)
    ratio = A / -(np.arange(w.N) + 1.0)[None, :]
    assert ratio.min() >= 0.5 and ratio.max() <= 1.5 and abs(ratio.mean() - 1.0) < 0.01


def test_decode_step_inputs():
    w = I.WORKLOADS["decode_bf16_b512_d4096_N16_x64"]
    s0 = I.decode_step_inputs(w, 0)
    s1 = I.decode_step_inputs(w, 1)
    assert s0["x"].shape == (512, 4096) and s0["x"].dtype == np.uint16
    assert s0["B"].shape == (512, 16)
    assert not np.array_equal(s0["x"], s1["x"])
    st = I.decode_initial_state(w)
    assert st.shape == (512, 4096, 16) and st.dtype == np.float32
    assert abs(float(st.std()) - 0.1) < 1e-3
