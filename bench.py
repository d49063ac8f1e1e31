#!/usr/bin/env python3
"""Throughput of the selective scan on one MI355X.

A step is one ssm_scan_fwd call over one batch of the long-context workload (b=1, d=2048,
L=131072, N=16, bf16 storage with an fp32 state, gate on, final state returned), the largest
configuration that runs on one GPU: ZOH discretisation, recurrence, readout, gate/skip epilogue, and
the chunk carry across time segments. Inputs are synthetic (seeded draws with the workload's
distributions) and resident in HBM before timing; where one set fits the 256 MB last-level cache,
several copies rotate.

Printed: one JSON line. `value` is GB/s of algorithmic traffic (inputs read once, outputs written
once) over the whole timed call; `roofline` describes the output-pass kernel, timed with HIP
events on the launch stream, against the VALU issue rate (the bound of an exact exp per (t, n)),
with the HBM and ALU fractions of the kernel and of the whole call beside it; `cpu_baseline` times the
fp64 oracle on the host; `extra` carries every other workload: the tiny one (µs per call), the
130M-like and 1.4B-like prefills, the decode steps, and the gradient, Conv1D, LTI and SSD forms.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                        # MI355X HBM3E, published
VALU_PEAK_TSLOT = 256 * 4 * 16 * 2.4e9 / 1e12  # 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz = 39.32 T lane-slots/s
MFMA_F32_PEAK_TFLOPS = 157.3                 # MI355X dense fp32 MFMA, published
MFMA_BF16_PEAK_TFLOPS = 2500.0               # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20
# The shader clock climbs to its sustained level over tens of milliseconds of back-to-back work, and
# drops while the GPU idles (as it does while inputs are generated on the host). A headline run with 5
# warm-up calls read 1.31-1.36 TB/s where 200 or more read 1.50-1.52 TB/s. Hence the default warm-up
# below, and a warm-up of at least EXTRA_WARM_S seconds before each extra measurement.
DEFAULT_WARMUP = 500
DEFAULT_STEPS = 500
EXTRA_WARM_S = 0.25
HEAD_WARM_S = 1.0
HEADLINE = "longctx_bf16_b1_d2048_L131072_N16"
# the machine's CPU share for one GPU; the oracle baseline uses at most this many host threads
HOST_THREAD_CAP = 16
GRAD_WORKLOAD = "mamba130m_f32_b4_d1536_L2048_N16"
SIDE_WORKLOADS = ("mamba130m_f32_b4_d1536_L2048_N16", "mamba1p4b_bf16_b8_d4096_L4096_N16")
DEFAULT_EXTRA = ("tiny_f32_b1_d8_L128_N4,mamba130m_f32_b4_d1536_L2048_N16,mamba1p4b_bf16_b8_d4096_L4096_N16,"
                 "decode,grad,conv,frontend,lti,ssd")
METRIC = "selective-scan GB/s & % of HBM peak; (b·d·L)/s at N=16; decode steps/s"


def valu_slots_per_element(N, gate):
    """Issue slots the method needs per (b, d, t) on CDNA4: per state one exp (2 slots, half rate)
    and six fp32 VALU operations (Δ·A; s + B·x; Ā − 1; the update FMA; C/A; the readout FMA); per
    element the skip FMA and, with the gate, silu and the product (mul, exp, add, rcp, mul, mul)."""
    return 8 * N + (1 + (8 if gate else 0))


def algorithmic_bytes(b, d, L, N, esize, gate, with_D=True, with_state=True):
    rows = b * d * L * esize
    return (rows * (3 if gate else 2) + rows            # x, delta, (z) read; y written
            + 2 * b * L * N * esize                      # B, C
            + d * N * 4 + (d * 4 if with_D else 0)       # A, D
            + (b * d * N * 4 if with_state else 0))      # final state


def to_dev(arr, dev):
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def warm_up(fn, count, min_s=0.0):
    """`count` untimed calls of fn(i), then more until min_s seconds have passed."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < count or time.perf_counter() - t0 < min_s:
        fn(i)
        i += 1
        if i % 8 == 0 and i >= count:
            torch.cuda.synchronize()  # keep the queue short, so the clock check follows the GPU
    torch.cuda.synchronize()


def bench_prefill(name, steps, warmup, rotate=0, quiet=False, min_warm_s=0.0, call_kw=None):
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    dev = torch.device("cuda:0")
    t_gen = time.time()
    inp = I.prefill_inputs(w)
    gen_s = time.time() - t_gen
    esize = 4 if w.dtype == "f32" else 2
    nbytes = algorithmic_bytes(w.b, w.d, w.L, w.N, esize, w.gate)
    if rotate <= 0:
        rotate = int(min(8, max(1, -(-2 * MALL_BYTES // nbytes))))
    sets = []
    for _ in range(rotate):
        s = {k: to_dev(inp[k], dev) for k in ("x", "delta", "z", "A", "B", "C", "D")}
        s["y"] = torch.empty_like(s["x"])
        s["h"] = torch.empty((w.b, w.d, w.N), dtype=torch.float32, device=dev)
        sets.append(s)
    # the output kernel is timed on every `every`-th call of the timed loop (each event pair adds a
    # few microseconds of queue drain to the call it brackets)
    every = max(1, steps // 10)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:  # materialise the underlying HIP events before handing them to the library
        e0.record(); e1.record()

    def call(i, events=None):
        s = sets[i % rotate]
        api.ssm_scan_fwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], y=s["y"], final_state=s["h"],
                         events=events, **(call_kw or {}))

    warm_up(call, warmup, min_warm_s)
    t0 = time.perf_counter()
    for i in range(steps):
        call(i, ev[i] if i % every == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    kern = np.array([a.elapsed_time(b) for i, (a, b) in enumerate(ev) if i % every == 0])
    kern_ms = float(np.mean(kern))
    plan = api.ssm_scan_fwd_plan(w.b, w.d, w.L, w.N, torch.float32 if w.dtype == "f32" else torch.bfloat16,
                                 **(call_kw or {}))
    elems = w.b * w.d * w.L
    slots = elems * valu_slots_per_element(w.N, w.gate)
    call_tslot = slots / (ms * 1e-3) / 1e12
    kern_tslot = slots / (kern_ms * 1e-3) / 1e12
    res = {
        "workload": name, "ms_per_call": ms, "us_per_call": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9,
        "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alu_frac": call_tslot / VALU_PEAK_TSLOT,
        "elements_per_s": elems / (ms * 1e-3),
        "output_kernel_ms": kern_ms, "output_kernel_samples": int(len(kern)),
        "output_kernel_ms_p10_p50_p90": [round(float(q), 5) for q in np.percentile(kern, [10, 50, 90])],
        "output_kernel_share_of_call": kern_ms / ms,
        "algorithmic_bytes": nbytes, "rotating_sets": rotate, "plan": plan,
        "valu_slots_per_element": valu_slots_per_element(w.N, w.gate),
        "call_valu_Tslot_s": call_tslot, "kernel_valu_Tslot_s": kern_tslot,
        "kernel_alu_frac": kern_tslot / VALU_PEAK_TSLOT,
        "kernel_GBps": nbytes / (kern_ms * 1e-3) / 1e9,
        "kernel_hbm_frac": nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "input_gen_s": gen_s,
        "warmup_calls": warmup, "min_warmup_s": min_warm_s,
    }
    if not quiet:
        print(f"# {name}: {ms * 1e3:.1f} us/call, {res['GBps']:.0f} GB/s ({res['hbm_frac']:.3f} HBM, "
              f"{res['alu_frac']:.3f} ALU), output kernel {kern_ms * 1e3:.1f} us ({res['kernel_alu_frac']:.3f} ALU), "
              f"plan {plan}", file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res, inp


def grad_slots_per_element(N, gate):
    """VALU issue slots of the gradient pass per (b, d, t): per state the forward recomputation
    (Δ·A, exp (2), β, B·x, the update: 8) and the walk back (Ā, β again: 5; λ; ∂L/∂Ā; ∂L/∂β (2);
    the dB and dC partials (3); the dx, dΔ and dA terms (2 + 2 + 5); the carried adjoint; the readout
    for dz: 23), plus per element the gate and its derivative (12) and the skip terms (3)."""
    return 31 * N + (15 if gate else 3)


def bench_grad(name, steps, warmup, quiet=False):
    """The gradient pass (ssm_scan_bwd) on a prefill workload: dy ~ N(0, 1) of y's shape."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    inp = I.prefill_inputs(w)
    esize = 4 if w.dtype == "f32" else 2
    rows = w.b * w.d * w.L
    # read x, Δ, z, dy, B, C, A, D; write dx, dΔ, dz, dA, dB, dC (fp32), dD
    nbytes = rows * esize * (4 if w.gate else 3) + rows * esize * (3 if w.gate else 2) \
        + 2 * w.b * w.L * w.N * esize + 2 * w.b * w.L * w.N * 4 + 2 * (w.d * w.N * 4 + w.d * 4)
    rotate = int(min(4, max(1, -(-2 * MALL_BYTES // nbytes))))
    rng = np.random.default_rng(5)
    sets = []
    for _ in range(rotate):
        s = {k: to_dev(inp[k], "cuda") for k in ("x", "delta", "z", "A", "B", "C", "D")}
        s["dy"] = to_dev(I.store(rng.standard_normal((w.b, w.d, w.L)), w.dtype), "cuda")
        sets.append(s)

    def call(i):
        s = sets[i % rotate]
        return api.ssm_scan_bwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], dy=s["dy"])

    warm_up(call, warmup, EXTRA_WARM_S)
    t0 = time.perf_counter()
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    slots = rows * grad_slots_per_element(w.N, w.gate)
    res = {"pass": "gradient", "workload": name, "ms_per_call": ms, "elements_per_s": rows / (ms * 1e-3),
           "GBps": nbytes / (ms * 1e-3) / 1e9, "algorithmic_bytes": nbytes,
           "valu_slots_per_element": grad_slots_per_element(w.N, w.gate),
           "call_valu_Tslot_s": slots / (ms * 1e-3) / 1e12,
           "call_valu_frac": slots / (ms * 1e-3) / 1e12 / VALU_PEAK_TSLOT}
    if not quiet:
        print(f"# gradient {name}: {ms * 1e3:.1f} us/call, {res['elements_per_s']:.3g} elements/s, "
              f"{res['call_valu_Tslot_s']:.2f} T VALU slot/s over the whole call", file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res


LTI_MAX_L = 8192   # one transform's sequence length (SSM_LTI_MAX_L)
LTI_CHUNK = 4096   # chunk length of the longer, chunked form (SSM_LTI_CHUNK)


def lti_fft_points(L):
    """Transform size of the LTI convolution for sequence length L (a power of two >= max(2L, 1024))."""
    m = 1024
    while m < 2 * L:
        m *= 2
    return m


def bench_lti(name, steps, warmup, quiet=False):
    """The time-invariant form (ssm_lti_fwd: K̄, then the FFT convolution) on a layer of the workload's
    shape with per-channel Δ, B, C (the LTI input recipe), gate and D on."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    inp = I.random_lti(w.b, w.d, w.L, w.N, dtype=w.dtype, gate=w.gate, seed=2)
    esize = 4 if w.dtype == "f32" else 2
    rows = w.b * w.d * w.L
    # beyond one transform, chunks of 4096 steps joined through the state (K̄ over 4096 taps)
    chunked = w.L > LTI_MAX_L
    klen = LTI_CHUNK if chunked else w.L
    n_chunks = -(-w.L // klen)
    # read x, z; write y; read the parameters; K̄ [d][klen] fp32 is written once and read once per chunk
    nbytes = rows * esize * (3 if w.gate else 2) + w.d * (3 * w.N + 2) * 4 + w.d * klen * 4 * (1 + n_chunks)
    M = lti_fft_points(klen)
    transforms = w.d * n_chunks * (1 + 2 * ((w.b + 1) // 2))
    flops = transforms * 5 * M * math.log2(M) + w.d * n_chunks * ((w.b + 1) // 2) * 6 * M  # radix-2 count
    rotate = int(min(8, max(1, -(-2 * MALL_BYTES // nbytes))))
    par = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda() for k in ("delta", "A", "B", "C", "D")}
    sets = []
    for _ in range(rotate):
        x = to_dev(inp["x"], "cuda")
        sets.append((x, to_dev(inp["z"], "cuda") if w.gate else None, torch.empty_like(x)))
    K = None if chunked else api.ssm_lti_kernel(par["delta"], par["A"], par["B"], par["C"], w.L)

    def timed(fn):
        warm_up(fn, warmup, EXTRA_WARM_S)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def full(i):
        x, z, y = sets[i % rotate]
        api.ssm_lti_fwd(x, par["delta"], par["A"], par["B"], par["C"], par["D"], z, y=y)

    def conv_only(i):
        x, z, y = sets[i % rotate]
        api.ssm_lti_conv(x, K, par["D"], z, y=y)

    ms = timed(full)
    # the convolution alone (a given K̄) exists for one transform; the chunked form is timed whole
    ms_conv = timed(conv_only) if not chunked else None
    res = {"pass": "lti_fft", "workload": name, "us_per_call": ms * 1e3,
           "us_conv_only": ms_conv * 1e3 if ms_conv else None, "chunked": chunked, "chunk": klen,
           "n_chunks": n_chunks, "elements_per_s": rows / (ms * 1e-3), "algorithmic_bytes": nbytes,
           "GBps": nbytes / (ms * 1e-3) / 1e9, "fft_points": M, "transforms": transforms,
           "fft_TFLOPs_call": flops / (ms * 1e-3) / 1e12,
           "fft_TFLOPs_conv": flops / (ms_conv * 1e-3) / 1e12 if ms_conv else None}
    if not quiet:
        conv_txt = f"convolution alone {ms_conv * 1e3:.1f} us" if ms_conv else f"{n_chunks} chunks of {klen} steps"
        print(f"# lti {name}: {ms * 1e3:.1f} us/call ({conv_txt}), {res['GBps']:.0f} GB/s, "
              f"{res['fft_TFLOPs_call']:.1f} TFLOP/s over the call (5 M log2 M per transform)",
              file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res


SSD_SHAPES = {  # name: (b, H, L, N, dtype); heads of 64 channels
    "ssd_f32_b4_H24_L2048_N64": (4, 24, 2048, 64, "f32"),
    "ssd_bf16_b8_H64_L4096_N128": (8, 64, 4096, 128, "bf16"),
}


def ssd_mfma_flops(b, H, L, N, P=64, Q=64):
    """fp32 MFMA flops the chunked form issues: per (b, head, chunk) the chunk state (2·P·N·Q), C·Bᵀ on the
    three tiles at or below the diagonal (3·2·32²·N), the decayed products times x (2·32²·(2·32 + 2·64)) and
    C times the entering state (2·Q·P·N)."""
    per = 2 * P * N * Q + 6 * 32 * 32 * N + 2 * 32 * 32 * 192 + 2 * Q * P * N
    return b * H * (-(-L // Q)) * per


def bench_ssd(name, steps, warmup, quiet=False):
    """The scalar-decay (state space duality) form, ssm_ssd_fwd, on a layer of the named shape; for N <= 64
    the recurrent kernel (ssm_scan_fwd with Δ repeated over each head and A = a_h) is timed beside it."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    b, H, L, N, dt = SSD_SHAPES[name]
    P = 64
    inp = I.random_ssd(b, H, L, N, dtype=dt, seed=2)
    es = 4 if dt == "f32" else 2
    d = H * P
    nbytes = b * d * L * es * 3 + b * H * L * es + 2 * b * L * N * es + b * d * N * 4 + d * 4 + H * 4
    # chunk states through HBM (written, read and rewritten by the pass, read): none for the single walk
    # (bf16 storage, N of 64 or 128, b·H at least twice the compute units)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    single_walk = dt == "bf16" and N in (64, 128) and b * H >= 2 * cus
    scratch_traffic = 0 if single_walk else 4 * b * H * (-(-L // 64)) * P * N * 4
    flops = ssd_mfma_flops(b, H, L, N)
    rotate = int(min(8, max(1, -(-2 * MALL_BYTES // nbytes))))
    sets = []
    for _ in range(rotate):
        t = {k: to_dev(inp[k], "cuda") for k in ("x", "z", "delta", "B", "C")}
        t["A"] = torch.from_numpy(inp["A"]).cuda()
        t["D"] = torch.from_numpy(inp["D"]).cuda()
        t["y"] = torch.empty_like(t["x"])
        t["h"] = torch.empty((b, d, N), device="cuda")
        sets.append(t)

    def timed(fn):
        warm_up(fn, warmup, EXTRA_WARM_S)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def ssd(i):
        t = sets[i % rotate]
        api.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], y=t["y"], final_state=t["h"])

    ms = timed(ssd)
    res = {"pass": "ssd_chunked_mfma", "workload": name, "us_per_call": ms * 1e3, "elements_per_s": b * d * L / (ms * 1e-3),
           "algorithmic_bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9, "scratch_bytes_moved": scratch_traffic,
           "single_walk": single_walk, "mfma_flops": flops, "mfma_TFLOPs": flops / (ms * 1e-3) / 1e12,
           "mfma_instruction": "f32_32x32x2" if dt == "f32" else "bf16_32x32x16 (fp32 operands as hi + lo)",
           "mfma_frac": flops / (ms * 1e-3) / 1e12 / (MFMA_F32_PEAK_TFLOPS if dt == "f32" else MFMA_BF16_PEAK_TFLOPS)}
    if N <= 64:
        for t in sets:
            t["dl"] = t["delta"].repeat_interleave(P, dim=1).contiguous()
            t["A2"] = t["A"].repeat_interleave(P)[:, None].expand(d, N).contiguous()

        def rec(i):
            t = sets[i % rotate]
            api.ssm_scan_fwd(t["x"], t["dl"], t["A2"], t["B"], t["C"], t["D"], t["z"], y=t["y"], final_state=t["h"])
        res["us_recurrent_kernel"] = timed(rec) * 1e3
    if not quiet:
        extra = f", recurrent kernel {res['us_recurrent_kernel']:.1f} us" if "us_recurrent_kernel" in res else ""
        print(f"# ssd {name}: {ms * 1e3:.1f} us/call, {res['GBps']:.0f} GB/s, {res['mfma_TFLOPs']:.1f} TFLOP/s of "
              f"matrix products ({res['mfma_instruction']}){extra}", file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res


def bench_conv(name, steps, warmup, W=4, quiet=False):
    """The Conv1D + SiLU front end over the workload's [b, d, L] input (taps N(0, 0.5²), bias N(0, 1)),
    returning the state; HBM-bound: algorithmic bytes = xin read + x written (+ taps, bias, state)."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    inp = I.prefill_inputs(w)
    esize = 4 if w.dtype == "f32" else 2
    rows = w.b * w.d * w.L
    nbytes = 2 * rows * esize + w.d * (W + 1) * 4 + w.b * w.d * (W - 1) * 4
    rotate = int(min(8, max(1, -(-2 * MALL_BYTES // nbytes))))
    rng = np.random.default_rng(6)
    taps = torch.from_numpy((rng.standard_normal((w.d, W)) * 0.5).astype(np.float32)).cuda()
    bias = torch.from_numpy(rng.standard_normal(w.d).astype(np.float32)).cuda()
    sets = []
    for _ in range(rotate):
        xin = to_dev(inp["x"], "cuda")
        sets.append((xin, torch.empty_like(xin), torch.empty((w.b, w.d, W - 1), device="cuda")))

    def call(i):
        xin, xo, so = sets[i % rotate]
        api.ssm_conv1d_fwd(xin, taps, bias, x_out=xo, state_out=so)

    warm_up(call, warmup, EXTRA_WARM_S)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res = {"pass": "conv1d", "workload": name, "W": W, "us_per_call": ms * 1e3, "algorithmic_bytes": nbytes,
           "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if not quiet:
        print(f"# conv1d {name} (W={W}): {ms * 1e3:.1f} us/call, {res['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res


def bench_frontend(name, steps, warmup, W=4, quiet=False):
    """The fused front end (ssm_scan_fwd_conv: Conv1D + SiLU folded into the scan's staging) against the two
    launches it replaces (ssm_conv1d_fwd, then ssm_scan_fwd on its output), on the workload's inputs with
    the Conv1D input standing in for x; and the fused call with Δ's bias and softplus applied inside."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    inp = I.prefill_inputs(w)
    esize = 4 if w.dtype == "f32" else 2
    nbytes = algorithmic_bytes(w.b, w.d, w.L, w.N, esize, w.gate) + w.d * (W + 1) * 4 + 2 * w.b * w.d * (W - 1) * 4
    rotate = int(min(8, max(1, -(-2 * MALL_BYTES // nbytes))))
    rng = np.random.default_rng(7)
    taps = torch.from_numpy((rng.standard_normal((w.d, W)) * 0.5).astype(np.float32)).cuda()
    cbias = torch.from_numpy(rng.standard_normal(w.d).astype(np.float32)).cuda()
    dbias = torch.from_numpy((rng.standard_normal(w.d) * 0.3).astype(np.float32)).cuda()
    sets = []
    for _ in range(rotate):
        t = {k: to_dev(inp[k], "cuda") for k in ("x", "delta", "z", "A", "B", "C", "D")}
        t["y"] = torch.empty_like(t["x"])
        t["xc"] = torch.empty_like(t["x"])
        t["h"] = torch.empty((w.b, w.d, w.N), device="cuda")
        t["cs_in"] = torch.zeros((w.b, w.d, W - 1), device="cuda")
        t["cs_out"] = torch.empty((w.b, w.d, W - 1), device="cuda")
        sets.append(t)

    def timed(fn):
        warm_up(fn, warmup, EXTRA_WARM_S)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def fused(i, softplus=False):
        t = sets[i % rotate]
        api.ssm_scan_fwd_conv(t["x"], taps, t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], conv_bias=cbias,
                              conv_state_in=t["cs_in"], delta_bias=dbias if softplus else None,
                              delta_softplus=softplus, y=t["y"], final_state=t["h"], conv_state_out=t["cs_out"])

    def pair(i):
        t = sets[i % rotate]
        api.ssm_conv1d_fwd(t["x"], taps, cbias, state_in=t["cs_in"], x_out=t["xc"], state_out=t["cs_out"])
        api.ssm_scan_fwd(t["xc"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], y=t["y"], final_state=t["h"])

    ms_pair = timed(pair)
    ms_fused = timed(fused)
    ms_fused_sp = timed(lambda i: fused(i, True))
    res = {"pass": "fused_frontend", "workload": name, "W": W, "us_two_launches": ms_pair * 1e3,
           "us_fused": ms_fused * 1e3, "us_fused_softplus": ms_fused_sp * 1e3, "speedup": ms_pair / ms_fused,
           "algorithmic_bytes_fused": nbytes, "GBps_fused": nbytes / (ms_fused * 1e-3) / 1e9}
    if not quiet:
        print(f"# fused front end {name} (W={W}): {ms_fused * 1e3:.1f} us fused ({ms_fused_sp * 1e3:.1f} us with Δ bias "
              f"and softplus) against {ms_pair * 1e3:.1f} us for Conv1D then scan", file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res


def bench_decode(name, rotate_states, quiet=False):
    """The decode workload: `steps` successive single-token steps, each with fresh inputs, on one
    state (rotate_states = 1, the literal workload) or cycling through several layer states."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    dev = torch.device("cuda:0")
    st0 = torch.from_numpy(I.decode_initial_state(w)).to(dev)
    states = [st0.clone() for _ in range(rotate_states)]
    stepin = []
    for s in range(w.steps):
        si = I.decode_step_inputs(w, s)
        stepin.append({k: to_dev(si[k], dev) for k in ("x", "delta", "z", "A", "B", "C", "D")})
    ys = [torch.empty((w.b, w.d), dtype=stepin[0]["x"].dtype, device=dev) for _ in range(2)]

    def step(i):
        t = stepin[i % w.steps]
        api.ssm_scan_step(states[i % rotate_states], t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                          y=ys[i % 2])

    warm_up(step, 4, EXTRA_WARM_S)
    for j, s in enumerate(states):
        s.copy_(st0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(w.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    esize = 2 if w.dtype == "bf16" else 4
    per_step = (2 * w.b * w.d * w.N * 4 + 4 * w.b * w.d * esize + 2 * w.b * w.N * esize + w.d * w.N * 4 + w.d * 4)
    per_step_s = gpu_ms * 1e-3 / w.steps
    res = {"workload": name, "states_rotated": rotate_states, "steps": w.steps,
           "steps_per_s": w.steps / (gpu_ms * 1e-3), "tokens_per_s": w.b * w.steps / (gpu_ms * 1e-3),
           "us_per_step": per_step_s * 1e6, "GBps": per_step / per_step_s / 1e9,
           "hbm_frac": per_step / per_step_s / 1e9 / HBM_PEAK_GBS, "bytes_per_step": per_step,
           "wall_steps_per_s": w.steps / wall}
    if not quiet:
        print(f"# {name} (states rotated: {rotate_states}): {res['us_per_step']:.1f} us/step, "
              f"{res['steps_per_s']:.0f} steps/s, {res['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    return res


def cpu_baseline(inp, name, threads, target_thread_s=15.0):
    """The fp64 oracle on the host over a bounded sample of the workload: blocks of 16 channels of a batch
    row over the whole sequence (each row is sequential in t), spread over `threads` host threads, as many
    blocks as make about `target_thread_s` seconds of CPU work (one block is timed alone first)."""
    import concurrent.futures as cf

    import oracle
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    dt = inp["dtype"]
    blk = 16
    chunks = [(ib, c0, min(w.d, c0 + blk)) for ib in range(w.b) for c0 in range(0, w.d, blk)]

    def one(job):
        ib, c0, c1 = job
        wd = lambda a: I.widen(a[ib:ib + 1, c0:c1], dt)
        oracle.scan_fwd(wd(inp["x"]), wd(inp["delta"]), inp["A"][c0:c1], I.widen(inp["B"][ib:ib + 1], dt),
                        I.widen(inp["C"][ib:ib + 1], dt), inp["D"][c0:c1],
                        None if inp["z"] is None else wd(inp["z"]))

    t0 = time.perf_counter()
    one(chunks[0])
    one_s = time.perf_counter() - t0
    n = int(target_thread_s / max(one_s, 1e-6))
    n = max(threads, min(len(chunks), (n // threads) * threads if n >= threads else threads))
    n = min(n, len(chunks))
    sample = chunks[:n]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, sample))
    wall = time.perf_counter() - t0
    rows = sum(c1 - c0 for _, c0, c1 in sample)
    elems = rows * w.L
    esize = 4 if dt == "f32" else 2
    per_elem = algorithmic_bytes(w.b, w.d, w.L, w.N, esize, w.gate) / (w.b * w.d * w.L)
    return {"value": elems * per_elem / wall / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of the workload's {w.b * w.d} (b,d) rows, each over all {w.L} steps x {w.N} states "
                      f"(fp64, sequential in t), on {threads} host threads: {wall:.2f} s wall, about "
                      f"{wall * threads:.0f} thread-s; GB/s counts the workload's algorithmic bytes per element",
            "host_cpu_count": os.cpu_count(),
            "thread_cap": f"{HOST_THREAD_CAP} (the host's CPU share for one GPU)",
            "elements_per_s": elems / wall,
            "single_thread_elements_per_s": (chunks[0][2] - chunks[0][1]) * w.L / one_s,
            "single_thread_sample": f"{chunks[0][2] - chunks[0][1]} (b,d) rows x {w.L} steps on one thread, {one_s:.3f} s"}


def bench_tiny_latency(name, calls=200):
    """Latency of one call on the tiny workload: host wall time of call + synchronize, per call (median)."""
    import torch
    from selective_state_space_82_amd import api
    from selective_state_space_82_amd import inputs as I

    w = I.WORKLOADS[name]
    inp = I.prefill_inputs(w)
    t = {k: to_dev(inp[k], "cuda") for k in ("x", "delta", "z", "A", "B", "C", "D")}
    y = torch.empty_like(t["x"])
    h = torch.empty((w.b, w.d, w.N), dtype=torch.float32, device="cuda")
    lat = []
    for i in range(calls + 20):
        t0 = time.perf_counter()
        api.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], y=y, final_state=h)
        torch.cuda.synchronize()
        if i >= 20:
            lat.append(time.perf_counter() - t0)
    return float(np.median(lat) * 1e6), [round(float(q) * 1e6, 2) for q in np.percentile(lat, [10, 90])]


def copy_bandwidth(nbytes=1 << 30, reps=5):
    """Device-to-device copy rate (GB/s, bytes read + written), the practical HBM ceiling."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def copy_probe(nbytes):
    """A plain device copy of known size (calibrates the HBM byte counters)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma list: 'decode', 'grad' (gradient pass on the 130M-like workload), 'conv' (Conv1D "
                         "front end), 'frontend' (Conv1D fused into the scan, against the two launches), 'lti' "
                         "(LTI convolution form), 'ssd' (scalar-decay chunked form) "
                         "and/or prefill workload names "
                         "('' for none, 'all' for every one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0, help="input/output sets to rotate (0 = enough to exceed the cache)")
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a plain copy of this many bytes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (the scan shards by batch row or "
              "channel with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    from selective_state_space_82_amd import inputs as I

    copy_gbps = copy_bandwidth()
    print(f"# device copy: {copy_gbps:.0f} GB/s (read + write)", file=sys.stderr, flush=True)
    head, inp = bench_prefill(args.workload, args.steps, args.warmup, args.rotate, min_warm_s=HEAD_WARM_S)
    w = I.WORKLOADS[args.workload]
    extra = []
    names = [n for n in args.extra.split(",") if n]
    if names == ["all"]:
        names = ["decode"] + [n for n in I.PREFILL_WORKLOADS if n != args.workload]
    for n in names:
        if n == "decode":
            for r in (1, 4):
                extra.append(bench_decode(I.DECODE_WORKLOADS[0], r))
        elif n == "grad":
            extra.append(bench_grad(GRAD_WORKLOAD, max(3, min(args.steps, 100)), 2))
        elif n == "ssd":
            for sn in SSD_SHAPES:
                extra.append(bench_ssd(sn, 20, 3))
        elif n == "lti":
            for cw in tuple(SIDE_WORKLOADS) + ("longctx_bf16_b1_d2048_L131072_N16",):
                extra.append(bench_lti(cw, 20, 3))
        elif n == "conv":
            for cw in SIDE_WORKLOADS:
                extra.append(bench_conv(cw, 20, 3))
        elif n == "frontend":
            extra.append(bench_frontend("mamba1p4b_bf16_b8_d4096_L4096_N16", 50, 3))
        elif n == args.workload:
            continue
        else:
            wl = I.WORKLOADS[n]
            small = wl.b * wl.d * wl.L < (1 << 20)
            r, _ = bench_prefill(n, 2000 if small else max(3, min(args.steps, 200)), 100 if small else 2,
                                 min_warm_s=EXTRA_WARM_S)
            if small:  # latency-bound: report the time of one call, back to back and synchronised
                r["us_per_call_synchronised"], r["us_per_call_synchronised_p10_p90"] = bench_tiny_latency(n)
                print(f"# {n}: {r['us_per_call']:.2f} us per call back to back, "
                      f"{r['us_per_call_synchronised']:.1f} us per synchronised call", file=sys.stderr, flush=True)
            extra.append(r)

    cpu = None
    if not args.no_cpu_baseline:
        threads = int(min(HOST_THREAD_CAP, os.cpu_count() or 1))
        cpu = cpu_baseline(inp, args.workload, threads)
        print(f"# cpu baseline: {cpu['value']:.3f} GB/s on {threads} threads", file=sys.stderr, flush=True)

    kern_s = head["output_kernel_ms"] * 1e-3
    slots = w.b * w.d * w.L * head["valu_slots_per_element"]
    traffic = None
    prof = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if os.path.exists(prof):
        try:
            from selective_state_space_82_amd import build as B
            with open(prof) as f:
                tc = json.load(f)
            if tc.get("kernel_source_sha256") == B.kernel_source_hash() and args.workload in tc.get("per_launch_bytes", {}):
                traffic = tc["per_launch_bytes"][args.workload]
        except Exception:  # a stale or unreadable counter file means no traffic figure
            traffic = None
    line = {
        "metric": METRIC,
        "value": round(head["GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_call"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Normal / softplus-Normal draws with the workload's distributions)",
        "config": {"workload": args.workload, "b": w.b, "d": w.d, "L": w.L, "N": w.N, "gate": w.gate,
                   "state": "f32", "plan": head["plan"], "rotating_sets": head["rotating_sets"],
                   "warmup": f"{args.warmup} calls and at least {HEAD_WARM_S} s"},
        "hbm_frac": round(head["hbm_frac"], 4),
        "alu_frac": round(head["alu_frac"], 4),
        "copy_GBps": round(copy_gbps, 1),
        "copy_frac": round(head["GBps"] / copy_gbps, 4),
        "elements_per_s": head["elements_per_s"],
        "roofline": {"bound": "alu", "achieved": round(slots / kern_s / 1e12, 3), "peak": round(VALU_PEAK_TSLOT, 3),
                     "unit": "Tslot/s", "frac": round(slots / kern_s / 1e12 / VALU_PEAK_TSLOT, 4),
                     "traffic": traffic, "kernel": "scan_fwd_kernel (output pass)",
                     "kernel_us": round(head["output_kernel_ms"] * 1e3, 2),
                     "kernel_us_p10_p50_p90": [round(q * 1e3, 2) for q in head["output_kernel_ms_p10_p50_p90"]],
                     "kernel_hbm_frac": round(head["kernel_hbm_frac"], 4),
                     "call_alu_frac": round(head["alu_frac"], 4), "call_hbm_frac": round(head["hbm_frac"], 4),
                     "kernel_share_of_call": round(head["output_kernel_share_of_call"], 4)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
