"""Seeded synthetic inputs for the selective scan (shared by the tests, the benchmark and smoke).

This module holds no arithmetic of the method itself: it draws random tensors with the shapes and
distributions of the Mamba-shaped workloads and quantises them to their storage type. The GPU path
and the oracle both consume its arrays; neither imports the other.

Storage conventions:
  * fp32 tensors are numpy float32 arrays.
  * bf16 tensors are numpy uint16 arrays holding the bf16 bit patterns, rounded from the fp64 draw
    to nearest-even in one step (round-to-odd through fp32, then nearest-even to bf16).
  * A and D are always fp32; the decode state is always fp32.
Layouts: x, delta, z, y [b][d][L]; A [d][N]; B, C [b][L][N]; D [d]; state [b][d][N].

Every tensor has its own generator, keyed by (seed, workload, tensor, chunk), so no tensor depends
on the order in which the others were drawn.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------------------------
# Workloads (Mamba-shaped synthetic layers; names carry their sizes)
# ---------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    d: int
    L: int            # sequence length (1 for the decode workload)
    N: int
    dtype: str        # "f32" or "bf16": storage type of x, delta, z, B, C, y
    gate: bool        # z present (y * silu(z))
    delta_mu: float   # delta = softplus(Normal(mu, sigma))
    delta_sigma: float
    a_kind: str       # "neg_index": A[d,n] = -(n+1); "neg_index_u": -(n+1) * U(0.5, 1.5)
    steps: int = 0    # decode workloads: number of successive single-token steps
    state_sigma: float = 0.0
    note: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_b1_d8_L128_N4", 1, 8, 128, 4, "f32", False, -2.0, 0.5, "neg_index",
                 note="tiny selective scan, gate off"),
        Workload("mamba130m_f32_b4_d1536_L2048_N16", 4, 1536, 2048, 16, "f32", True, -3.0, 1.0,
                 "neg_index", note="Mamba-130M-like layer scan, fp32, gate on"),
        Workload("mamba1p4b_bf16_b8_d4096_L4096_N16", 8, 4096, 4096, 16, "bf16", True, -2.0, 0.5,
                 "neg_index", note="Mamba-1.4B-like layer scan, bf16 in/out, fp32 state, gate on"),
        Workload("longctx_bf16_b1_d2048_L131072_N16", 1, 2048, 131072, 16, "bf16", True, -4.0, 1.0,
                 "neg_index_u", note="long-context scan, bf16 in/out, fp32 state carried in chunks"),
        Workload("decode_bf16_b512_d4096_N16_x64", 512, 4096, 1, 16, "bf16", True, -2.0, 0.5,
                 "neg_index", steps=64, state_sigma=0.1,
                 note="recurrent decode: 64 single-token steps, fp32 state in HBM"),
    ]
}

PREFILL_WORKLOADS = [n for n, w in WORKLOADS.items() if w.steps == 0]
DECODE_WORKLOADS = [n for n, w in WORKLOADS.items() if w.steps > 0]

_TENSOR_IDS = {"x": 1, "delta": 2, "z": 3, "A": 4, "B": 5, "C": 6, "D": 7, "state": 8, "A_u": 9}
_CHUNK_ROWS = 256


def _key(*parts) -> list[int]:
    h = hashlib.sha256(("/".join(str(p) for p in parts)).encode()).digest()
    return [int.from_bytes(h[i:i + 4], "little") for i in range(0, 16, 4)]


def _gen(seed, workload, tensor, *chunk) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(_key(seed, workload, tensor, *chunk))))


# ---------------------------------------------------------------------------------------------
# Storage quantisation
# ---------------------------------------------------------------------------------------------
def bf16_bits_from_f64(v) -> np.ndarray:
    """Round float64 values to bf16 (nearest-even, one rounding) and return the uint16 bits.

    fp64 -> fp32 is done round-to-odd (truncate, then set the lowest bit when inexact); fp32 keeps
    16 more bits than bf16, so the following nearest-even step rounds exactly as a direct
    fp64 -> bf16 rounding would. Finite inputs only."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    bits = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != v
    overshoot = inexact & (np.abs(f.astype(np.float64)) > np.abs(v))
    bits[overshoot] -= np.uint32(1)           # step the magnitude back toward zero (truncation)
    bits[inexact] |= np.uint32(1)             # sticky bit: round-to-odd
    rounding = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((bits + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(v, dtype: str) -> np.ndarray:
    """Quantise float64 values to the storage type ('f32' -> float32, 'bf16' -> uint16 bits)."""
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f64(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def widen(arr, dtype: str) -> np.ndarray:
    """Exact value of a stored tensor as float64."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _softplus(v):
    # input recipe only: the scan consumes delta as given
    return np.logaddexp(0.0, v)


# ---------------------------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------------------------
def _rows_tensor(seed, wname, tensor, b, d, L, dtype, draw, threads):
    """[b][d][L] tensor drawn in chunks of _CHUNK_ROWS channels, each from its own generator."""
    out = np.empty((b, d, L), dtype=np.float32 if dtype == "f32" else np.uint16)
    jobs = [(ib, c0) for ib in range(b) for c0 in range(0, d, _CHUNK_ROWS)]

    def one(job):
        ib, c0 = job
        c1 = min(d, c0 + _CHUNK_ROWS)
        g = _gen(seed, wname, tensor, ib, c0)
        out[ib, c0:c1] = store(draw(g, (c1 - c0, L)), dtype)

    if threads > 1 and len(jobs) > 1:
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out


def _a_matrix(seed, wname, d, N, a_kind):
    base = -(np.arange(N, dtype=np.float64) + 1.0)[None, :].repeat(d, axis=0)
    if a_kind == "neg_index":
        return base.astype(np.float32)
    if a_kind == "neg_index_u":
        u = _gen(seed, wname, "A_u").uniform(0.5, 1.5, size=(d, N))
        return (base * u).astype(np.float32)
    raise ValueError(a_kind)


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def prefill_inputs(w: Workload | str, seed: int = 0, threads: int | None = None) -> dict:
    """All inputs of one prefill call of workload `w` (storage form; see the module doc)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    threads = _threads() if threads is None else threads
    name = w.name
    normal = lambda g, shape: g.standard_normal(shape)
    dl = lambda g, shape: _softplus(g.normal(w.delta_mu, w.delta_sigma, size=shape))
    out = {
        "x": _rows_tensor(seed, name, "x", w.b, w.d, w.L, w.dtype, normal, threads),
        "delta": _rows_tensor(seed, name, "delta", w.b, w.d, w.L, w.dtype, dl, threads),
        "z": _rows_tensor(seed, name, "z", w.b, w.d, w.L, w.dtype, normal, threads) if w.gate else None,
        "A": _a_matrix(seed, name, w.d, w.N, w.a_kind),
        "B": store(_gen(seed, name, "B").standard_normal((w.b, w.L, w.N)), w.dtype),
        "C": store(_gen(seed, name, "C").standard_normal((w.b, w.L, w.N)), w.dtype),
        "D": _gen(seed, name, "D").standard_normal(w.d).astype(np.float32),
        "dtype": w.dtype,
        "shape": (w.b, w.d, w.L, w.N),
    }
    return out


def decode_initial_state(w: Workload | str, seed: int = 0) -> np.ndarray:
    """Initial fp32 state [b][d][N] ~ Normal(0, state_sigma) of a decode workload."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = _gen(seed, w.name, "state")
    return (g.standard_normal((w.b, w.d, w.N)) * w.state_sigma).astype(np.float32)


def decode_step_inputs(w: Workload | str, step: int, seed: int = 0) -> dict:
    """Inputs of decode step `step`: x, delta, z [b][d]; B, C [b][N]; D [d]; A [d][N]."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    name = w.name
    shp = (w.b, w.d)
    out = {
        "x": store(_gen(seed, name, "x", step).standard_normal(shp), w.dtype),
        "delta": store(_softplus(_gen(seed, name, "delta", step).normal(w.delta_mu, w.delta_sigma, size=shp)),
                       w.dtype),
        "z": store(_gen(seed, name, "z", step).standard_normal(shp), w.dtype) if w.gate else None,
        "A": _a_matrix(seed, name, w.d, w.N, w.a_kind),
        "B": store(_gen(seed, name, "B", step).standard_normal((w.b, w.N)), w.dtype),
        "C": store(_gen(seed, name, "C", step).standard_normal((w.b, w.N)), w.dtype),
        "D": _gen(seed, name, "D", step).standard_normal(w.d).astype(np.float32),
        "dtype": w.dtype,
        "shape": (w.b, w.d, w.N),
    }
    return out


def random_prefill(b, d, L, N, dtype="f32", gate=True, seed=0, delta_mu=-3.0, delta_sigma=1.0,
                   a_kind="neg_index", with_D=True, a_zero_frac=0.0, a_value=None, delta_value=None) -> dict:
    """Small random prefill inputs with the Mamba-shaped distributions, for edge-case tests.
    a_kind: "neg_index" (-(n+1)), "neg_index_u" (-(n+1)·U(0.5, 1.5)), "random" (-U(0.05, 4)) or
    "small" (-U(2^-10, 0.05), the regime where Δ·A is small). a_value / delta_value, when given, make
    A / Δ that constant everywhere. a_zero_frac > 0 sets that fraction of A entries to exactly 0 (the
    ZOH limit case)."""
    tag = f"random_{b}_{d}_{L}_{N}_{dtype}_{int(gate)}_{delta_mu}_{delta_sigma}_{a_kind}_{a_zero_frac}"
    if a_value is not None or delta_value is not None:
        tag += f"_{a_value}_{delta_value}"
    g = lambda t: _gen(seed, tag, t)
    if a_value is not None:
        A = np.full((d, N), a_value, dtype=np.float32)
    elif a_kind == "random":
        A = (-g("A").uniform(0.05, 4.0, size=(d, N))).astype(np.float32)
    elif a_kind == "small":
        A = (-g("A").uniform(2.0 ** -10, 0.05, size=(d, N))).astype(np.float32)
    else:
        A = _a_matrix(seed, tag, d, N, a_kind)
    if a_zero_frac > 0:
        mask = g("A0").uniform(size=(d, N)) < a_zero_frac
        A = np.where(mask, np.float32(0.0), A).astype(np.float32)
    if delta_value is not None:
        delta = store(np.full((b, d, L), float(delta_value)), dtype)
    else:
        delta = store(_softplus(g("delta").normal(delta_mu, delta_sigma, size=(b, d, L))), dtype)
    return {
        "x": store(g("x").standard_normal((b, d, L)), dtype),
        "delta": delta,
        "z": store(g("z").standard_normal((b, d, L)), dtype) if gate else None,
        "A": A,
        "B": store(g("B").standard_normal((b, L, N)), dtype),
        "C": store(g("C").standard_normal((b, L, N)), dtype),
        "D": g("D").standard_normal(d).astype(np.float32) if with_D else None,
        "dtype": dtype,
        "shape": (b, d, L, N),
    }


def random_lti(b, d, L, N, dtype="f32", gate=True, seed=0, delta_mu=-3.0, delta_sigma=1.0, with_D=True,
               a_zero_frac=0.0) -> dict:
    """Inputs of the time-invariant (convolution) form: every channel its own system.
    x, z [b][d][L] in storage form; delta [d] = softplus(N(mu, sigma)); A [d][N] = -(n+1); B, C [d][N]
    and D [d] ~ N(0, 1); all parameters fp32. a_zero_frac > 0 zeroes that fraction of A (the ZOH limit)."""
    tag = f"lti_{b}_{d}_{L}_{N}_{dtype}_{int(gate)}_{delta_mu}_{delta_sigma}_{a_zero_frac}"
    g = lambda t: _gen(seed, tag, t)
    A = _a_matrix(seed, tag, d, N, "neg_index")
    if a_zero_frac > 0:
        A = np.where(g("A0").uniform(size=(d, N)) < a_zero_frac, np.float32(0.0), A).astype(np.float32)
    return {
        "x": store(g("x").standard_normal((b, d, L)), dtype),
        "z": store(g("z").standard_normal((b, d, L)), dtype) if gate else None,
        "delta": _softplus(g("delta").normal(delta_mu, delta_sigma, size=d)).astype(np.float32),
        "A": A,
        "B": g("B").standard_normal((d, N)).astype(np.float32),
        "C": g("C").standard_normal((d, N)).astype(np.float32),
        "D": g("D").standard_normal(d).astype(np.float32) if with_D else None,
        "dtype": dtype,
        "shape": (b, d, L, N),
    }


def random_ssd(b, H, L, N, dtype="f32", gate=True, seed=0, delta_mu=-3.0, delta_sigma=1.0, with_D=True,
               a_zero_heads=(), P=64) -> dict:
    """Inputs of the scalar-decay (state space duality) form: H heads of P channels.
    x, z [b][H·P][L] and delta [b][H][L] = softplus(N(mu, sigma)) in storage form; B, C [b][L][N] ~ N(0, 1)
    in storage form; A [H] = -(h mod 16 + 1) fp32 (0 for the heads listed in a_zero_heads); D [H·P] ~ N(0, 1)."""
    tag = f"ssd_{b}_{H}_{L}_{N}_{P}_{dtype}_{int(gate)}_{delta_mu}_{delta_sigma}"
    g = lambda t: _gen(seed, tag, t)
    A = -((np.arange(H) % 16) + 1.0)
    for h in a_zero_heads:
        A[h] = 0.0
    return {
        "x": store(g("x").standard_normal((b, H * P, L)), dtype),
        "z": store(g("z").standard_normal((b, H * P, L)), dtype) if gate else None,
        "delta": store(_softplus(g("delta").normal(delta_mu, delta_sigma, size=(b, H, L))), dtype),
        "A": A.astype(np.float32),
        "B": store(g("B").standard_normal((b, L, N)), dtype),
        "C": store(g("C").standard_normal((b, L, N)), dtype),
        "D": g("D").standard_normal(H * P).astype(np.float32) if with_D else None,
        "dtype": dtype,
        "shape": (b, H, P, L, N),
    }


def random_frontend(b, d, L, N, W=4, dtype="f32", gate=True, seed=0, delta_mu=-3.0, delta_sigma=1.0,
                    a_kind="neg_index", with_state=True, with_h0=False) -> dict:
    """Inputs of the fused front end (Conv1D + SiLU, Δ bias and softplus, then the scan): the Conv1D's raw
    input xin ~ N(0, 1); raw Δ (before its bias and softplus) ~ N(mu, sigma); taps ~ N(0, 0.5²) [d][W];
    Conv1D bias ~ N(0, 1); Δ bias ~ N(0, 0.3²); the Conv1D state [b][d][W-1] ~ N(0, 1) and an initial SSM
    state [b][d][N] ~ N(0, 0.5²) when asked; A, B, C, D, z as in random_prefill."""
    tag = f"frontend_{b}_{d}_{L}_{N}_{W}_{dtype}_{int(gate)}_{delta_mu}_{delta_sigma}_{a_kind}"
    g = lambda t: _gen(seed, tag, t)
    return {
        "xin": store(g("xin").standard_normal((b, d, L)), dtype),
        "delta": store(g("delta").normal(delta_mu, delta_sigma, size=(b, d, L)), dtype),
        "z": store(g("z").standard_normal((b, d, L)), dtype) if gate else None,
        "A": _a_matrix(seed, tag, d, N, a_kind),
        "B": store(g("B").standard_normal((b, L, N)), dtype),
        "C": store(g("C").standard_normal((b, L, N)), dtype),
        "D": g("D").standard_normal(d).astype(np.float32),
        "conv_w": (g("conv_w").standard_normal((d, W)) * 0.5).astype(np.float32),
        "conv_bias": g("conv_bias").standard_normal(d).astype(np.float32),
        "delta_bias": (g("delta_bias").standard_normal(d) * 0.3).astype(np.float32),
        "conv_state": g("conv_state").standard_normal((b, d, W - 1)).astype(np.float32) if with_state else None,
        "h0": (g("h0").standard_normal((b, d, N)) * 0.5).astype(np.float32) if with_h0 else None,
        "dtype": dtype,
        "shape": (b, d, L, N, W),
    }
