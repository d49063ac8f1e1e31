"""GPU parity of the scalar-decay (state space duality) form, ssm_ssd_fwd through the C ABI, against the
fp64 oracle: the recurrent scan oracle_scan_fwd run with each head's Δ repeated over its channels and
A = a_h on every state (which the oracle pins tie to the quadratic masked-attention form).

Bar: |y - y_ref| <= τ·(1 + |y_ref|) element by element and the same for final states; τ = 1e-4 for fp32
storage, 2e-2 for bf16 storage.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TAU, from_torch, to_torch
from selective_state_space_82_amd import api
from selective_state_space_82_amd import inputs as I

pytestmark = pytest.mark.gpu
P = 64


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    api.lib()


def _upload(inp):
    dt, dev = inp["dtype"], torch.device("cuda:0")
    out = {k: to_torch(inp[k], dt, dev) for k in ("x", "z", "delta", "B", "C")}
    out["A"] = torch.from_numpy(inp["A"]).to(dev)
    out["D"] = None if inp["D"] is None else torch.from_numpy(inp["D"]).to(dev)
    return out


def _oracle_rows(inp, rows, h0=None):
    """Oracle y [len(rows), L] and final state [len(rows), N] for the (b, channel) pairs in rows."""
    dt = inp["dtype"]
    b, d, L = inp["x"].shape
    N = inp["B"].shape[2]
    w = lambda k: None if inp[k] is None else I.widen(inp[k], dt)
    x, z, dl, B, C = w("x"), w("z"), w("delta"), w("B"), w("C")
    ys, hs = [], []
    for ib, ch in rows:
        hh = ch // P
        yr, hr = oracle.scan_fwd(x[ib:ib + 1, ch:ch + 1], dl[ib:ib + 1, hh:hh + 1], np.full((1, N), inp["A"][hh]),
                                 B[ib:ib + 1], C[ib:ib + 1], None if inp["D"] is None else inp["D"][ch:ch + 1],
                                 None if z is None else z[ib:ib + 1, ch:ch + 1],
                                 None if h0 is None else h0[ib:ib + 1, ch:ch + 1].astype(np.float64))
        ys.append(yr[0, 0]); hs.append(hr[0, 0])
    return np.stack(ys), np.stack(hs)


def _close(got, ref, tau, what):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    print(f"[ssd] {what}: max err {worst:.2e}", flush=True)
    assert worst <= tau, f"{what}: max rel err {worst:.3e} > {tau} at {np.unravel_index(err.argmax(), err.shape)}"


def run_case(inp, h0=None, rows=None, what=""):
    t = _upload(inp)
    y, hT = api.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            initial_state=None if h0 is None else torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    b, d, L = inp["x"].shape
    if rows is None:
        rows = [(ib, ch) for ib in range(b) for ch in range(d)]
    yr, hr = _oracle_rows(inp, rows, h0)
    yg, hg = from_torch(y), from_torch(hT)
    tau = TAU[inp["dtype"]]
    _close(np.stack([yg[ib, ch] for ib, ch in rows]), yr, tau, f"{what} y")
    _close(np.stack([hg[ib, ch] for ib, ch in rows]), hr, tau, f"{what} final state")


CASES = [
    # b, H, L, N, dtype, gate, D, initial state, heads with a = 0
    (1, 1, 1, 32, "f32", False, False, False, ()),
    (2, 2, 64, 64, "f32", True, True, True, ()),       # exactly one chunk
    (1, 3, 100, 32, "f32", True, True, False, (1,)),   # ragged second chunk, a = 0 head
    (2, 1, 130, 128, "bf16", True, True, True, ()),
    (1, 2, 257, 64, "bf16", True, False, False, ()),
    (2, 2, 1000, 64, "f32", True, True, True, (0,)),   # 16 chunks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}_H{c[1]}_L{c[2]}_N{c[3]}_{c[4]}")
def test_ssd_matches_oracle(case):
    b, H, L, N, dt, gate, with_D, h0_on, a0 = case
    inp = I.random_ssd(b, H, L, N, dtype=dt, gate=gate, with_D=with_D, seed=L + N, a_zero_heads=a0)
    h0 = (np.random.default_rng(L).standard_normal((b, H * P, N)) * 0.5).astype(np.float32) if h0_on else None
    run_case(inp, h0, what=f"b{b} H{H} L{L} N{N} {dt}")


def test_ssd_empty_sequence():
    """L = 0: no output; the final state is the initial state (or zero)."""
    inp = I.random_ssd(1, 2, 0, 64, seed=3)
    t = _upload(inp)
    h0 = torch.randn(1, 2 * P, 64, device="cuda")
    _, hT = api.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], initial_state=h0)
    _, hz = api.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"])
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)
    assert torch.count_nonzero(hz) == 0


def test_ssd_matches_recurrent_scan_kernel():
    """The chunked MFMA form and the recurrent kernel ssm_scan_fwd (Δ repeated over each head, A = a_h
    on every state) agree, outputs and final states."""
    b, H, L, N = 2, 2, 700, 64
    inp = I.random_ssd(b, H, L, N, dtype="f32", seed=9)
    t = _upload(inp)
    y1, h1 = api.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"])
    dl = t["delta"].repeat_interleave(P, dim=1).contiguous()
    A2 = t["A"].repeat_interleave(P)[:, None].expand(H * P, N).contiguous()
    y2, h2 = api.ssm_scan_fwd(t["x"], dl, A2, t["B"], t["C"], t["D"], t["z"])
    torch.cuda.synchronize()
    _close(from_torch(y1), from_torch(y2), 2 * TAU["f32"], "SSD vs recurrent kernel y")
    _close(from_torch(h1), from_torch(h2), 2 * TAU["f32"], "SSD vs recurrent kernel state")


# On a 256-CU device: bf16 shapes with b·H >= 512 take the single-walk form (ssd_fused_kernel); other
# shapes with b·H·N/64 >= 512 take the fused state walk (ssd_scan_kernel) with the output kernel; the
# cases above take the three-kernel form. Ragged last chunks, initial states, both storage types. The
# single walk has three access modes: whole chunks (L a multiple of 64), whole 8-step pieces (L a
# multiple of 8) and element by element.
FUSED = [
    # b, H, L, N, dtype, initial state
    (8, 64, 130, 64, "f32", True),      # state walk
    (4, 128, 200, 128, "bf16", True),   # single walk, whole pieces, ragged last chunk
    (4, 128, 256, 128, "bf16", True),   # single walk, whole chunks, initial state
    (2, 256, 192, 64, "bf16", True),    # single walk, whole chunks, N = 64
    (8, 64, 64, 64, "bf16", False),     # single walk, one whole chunk (whole-chunk mode)
    (4, 64, 333, 128, "f32", False),    # state walk
    (4, 64, 150, 128, "bf16", True),    # state walk (b·H = 256)
    (2, 256, 104, 64, "bf16", False),   # single walk, N = 64, ragged last chunk
    (4, 128, 99, 64, "bf16", True),     # single walk, L not a multiple of 8 (element-wise edges)
    (4, 128, 1, 64, "bf16", True),      # single walk, one step
    (8, 64, 1, 64, "f32", True),        # state walk, one step
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"b{c[0]}_H{c[1]}_L{c[2]}_N{c[3]}_{c[4]}_h0{int(c[5])}")
def test_ssd_fused_state_walk(case):
    b, H, L, N, dt, h0_on = case
    inp = I.random_ssd(b, H, L, N, dtype=dt, seed=L + 7 * N, a_zero_heads=(3,))
    h0 = (np.random.default_rng(L + 1).standard_normal((b, H * P, N)) * 0.5).astype(np.float32) if h0_on else None
    rng = np.random.default_rng(L)
    rows = [(0, 0), (b - 1, H * P - 1), (0, 3 * P + 5)] + \
           [(int(rng.integers(b)), int(rng.integers(H * P))) for _ in range(60)]
    run_case(inp, h0, rows=rows, what=f"fused b{b} H{H} L{L} N{N} {dt}")


@pytest.mark.parametrize("shape", [(4, 24, 2048, 64, "f32"), (8, 64, 4096, 128, "bf16")],
                         ids=["b4_H24_L2048_N64_f32", "b8_H64_L4096_N128_bf16"])
def test_ssd_full_size_sampled(shape):
    """Full-size layers (d = H·64 = 1536 and 4096 channels) in the launch configuration the benchmark
    times, checked on sampled rows."""
    b, H, L, N, dt = shape
    inp = I.random_ssd(b, H, L, N, dtype=dt, seed=1)
    rng = np.random.default_rng(5)
    rows = [(0, 0), (b - 1, H * P - 1)] + [(int(rng.integers(b)), int(rng.integers(H * P))) for _ in range(20)]
    run_case(inp, rows=rows, what=f"full size {shape}")
