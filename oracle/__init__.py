"""fp64 sequential oracle of the selective state-space scan (ctypes wrapper over ssm_oracle.c).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package. The GPU library never loads it, and it imports nothing
from the GPU package: the two share no code.

Every array goes in and comes out as float64 (bf16 and fp32 inputs widen to float64 exactly).
Layouts follow the C header: x, delta, z, y are [b, d, L]; A is [d, N]; B, C are [b, L, N];
D is [d]; states are [b, d, N].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssm_oracle.c")
LIB_PATH = os.path.join(_HERE, "libssm_oracle.so")

_DP = ctypes.POINTER(ctypes.c_double)


def compile_library(src: str, out: str) -> str:
    """gcc build of an oracle source file into a shared library (always recompiles)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile the oracle library in place. Returns its path."""
    return compile_library(SOURCE, LIB_PATH)


def _f64(a, shape=None):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {arr.shape}")
    return arr


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_DP)


class Oracle:
    """The oracle's entry points bound to one compiled library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(lib_path)
        L = ctypes.c_long
        lib.oracle_scan_fwd.argtypes = [_DP] * 10 + [L, L, L, L]
        lib.oracle_scan_fwd.restype = ctypes.c_int
        lib.oracle_scan_step.argtypes = [_DP] * 9 + [L, L, L]
        lib.oracle_scan_step.restype = ctypes.c_int
        lib.oracle_scan_bwd.argtypes = [_DP] * 18 + [L, L, L, L]
        lib.oracle_scan_bwd.restype = ctypes.c_int
        lib.oracle_conv1d.argtypes = [_DP, _DP, _DP, _DP, ctypes.c_int, _DP, _DP, L, L, L, L]
        lib.oracle_conv1d.restype = ctypes.c_int
        lib.oracle_zoh.argtypes = [ctypes.c_double, ctypes.c_double, _DP, _DP]
        lib.oracle_lti_kernel.argtypes = [_DP] * 5 + [L, L, L]
        lib.oracle_lti_kernel.restype = ctypes.c_int
        lib.oracle_lti_conv.argtypes = [_DP] * 5 + [L, L, L]
        lib.oracle_lti_conv.restype = ctypes.c_int
        lib.oracle_ssd_quadratic.argtypes = [_DP] * 8 + [L, L, L, L, L]
        lib.oracle_ssd_quadratic.restype = ctypes.c_int
        lib.oracle_zoh.restype = None
        self.lib = lib
        self.path = lib_path

    def zoh(self, delta: float, a: float):
        """(Ā, bcoef) for one diagonal entry, with B̄ = bcoef · B."""
        ab = ctypes.c_double()
        bc = ctypes.c_double()
        self.lib.oracle_zoh(float(delta), float(a), ctypes.byref(ab), ctypes.byref(bc))
        return ab.value, bc.value

    def scan_fwd(self, x, delta, A, B, C, D=None, z=None, h0=None):
        """Prefill: returns (y [b, d, L], h_final [b, d, N]), both float64."""
        x = _f64(x)
        if x.ndim != 3:
            raise ValueError("x must be [b, d, L]")
        b, d, L = x.shape
        A = _f64(A)
        if A.ndim != 2:
            raise ValueError("A must be [d, N]")
        N = A.shape[1]
        delta = _f64(delta, (b, d, L))
        A = _f64(A, (d, N))
        B = _f64(B, (b, L, N))
        C = _f64(C, (b, L, N))
        D = _f64(D, (d,))
        z = _f64(z, (b, d, L))
        h0 = _f64(h0, (b, d, N))
        y = np.empty((b, d, L), dtype=np.float64)
        h = np.empty((b, d, N), dtype=np.float64)
        rc = self.lib.oracle_scan_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(z), _ptr(h0), _ptr(y), _ptr(h), b, d, L, N)
        if rc != 0:
            raise ValueError("oracle_scan_fwd rejected its arguments")
        return y, h

    def scan_bwd(self, x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_final=None):
        """Gradients of scan_fwd: a dict of float64 arrays dx, ddelta, dA, dB, dC, dD, dz, dh0
        (dD / dz are None when D / z are absent)."""
        x = _f64(x)
        b, d, L = x.shape
        A = _f64(A)
        N = A.shape[1]
        delta = _f64(delta, (b, d, L))
        B = _f64(B, (b, L, N))
        C = _f64(C, (b, L, N))
        D = _f64(D, (d,))
        z = _f64(z, (b, d, L))
        h0 = _f64(h0, (b, d, N))
        dy = _f64(dy, (b, d, L))
        dh_final = _f64(dh_final, (b, d, N))
        out = {"dx": np.empty((b, d, L)), "ddelta": np.empty((b, d, L)), "dA": np.empty((d, N)),
               "dB": np.empty((b, L, N)), "dC": np.empty((b, L, N)),
               "dD": None if D is None else np.empty(d), "dz": None if z is None else np.empty((b, d, L)),
               "dh0": np.empty((b, d, N))}
        rc = self.lib.oracle_scan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(out["dx"]),
                                      _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                                      _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["dh0"]), b, d, L, N)
        if rc != 0:
            raise ValueError("oracle_scan_bwd rejected its arguments")
        return out

    def conv1d(self, xin, w, bias=None, state=None, silu=True):
        """Causal depthwise Conv1D (+ SiLU): returns (x [b, d, L], new_state [b, d, W-1])."""
        xin = _f64(xin)
        b, d, L = xin.shape
        w = _f64(w)
        W = w.shape[1]
        w = _f64(w, (d, W))
        bias = _f64(bias, (d,))
        state = _f64(state, (b, d, W - 1))
        x = np.empty((b, d, L))
        st = np.empty((b, d, max(W - 1, 0)))
        rc = self.lib.oracle_conv1d(_ptr(xin), _ptr(w), _ptr(bias), _ptr(state), int(bool(silu)), _ptr(x),
                                    _ptr(st) if W > 1 else None, b, d, L, W)
        if rc != 0:
            raise ValueError("oracle_conv1d rejected its arguments")
        return x, st

    def scan_step(self, state, x, delta, A, B, C, D=None, z=None):
        """Decode step: returns (y [b, d], new_state [b, d, N]); `state` itself is not modified."""
        st = np.array(_f64(state), dtype=np.float64, copy=True)
        if st.ndim != 3:
            raise ValueError("state must be [b, d, N]")
        b, d, N = st.shape
        x = _f64(x, (b, d))
        delta = _f64(delta, (b, d))
        A = _f64(A, (d, N))
        B = _f64(B, (b, N))
        C = _f64(C, (b, N))
        D = _f64(D, (d,))
        z = _f64(z, (b, d))
        y = np.empty((b, d), dtype=np.float64)
        rc = self.lib.oracle_scan_step(_ptr(st), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                       _ptr(D), _ptr(z), _ptr(y), b, d, N)
        if rc != 0:
            raise ValueError("oracle_scan_step rejected its arguments")
        return y, st


    def lti_kernel(self, delta, A, B, C, L):
        """K̄ [d, L] of the time-invariant system per channel (delta [d]; A, B, C [d, N])."""
        A = _f64(A)
        if A.ndim != 2:
            raise ValueError("A must be [d, N]")
        d, N = A.shape
        delta = _f64(delta, (d,))
        B = _f64(B, (d, N))
        C = _f64(C, (d, N))
        K = np.empty((d, int(L)), dtype=np.float64)
        if self.lib.oracle_lti_kernel(_ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(K), d, int(L), N) != 0:
            raise ValueError("oracle_lti_kernel rejected its arguments")
        return K

    def lti_conv(self, x, K, D=None, z=None):
        """y [b, d, L] = causal x ∗ K̄ + D·x, times silu(z) when z is given."""
        x = _f64(x)
        if x.ndim != 3:
            raise ValueError("x must be [b, d, L]")
        b, d, L = x.shape
        K = _f64(K, (d, L))
        D = _f64(D, (d,))
        z = _f64(z, (b, d, L))
        y = np.empty_like(x)
        if self.lib.oracle_lti_conv(_ptr(x), _ptr(K), _ptr(D), _ptr(z), _ptr(y), b, d, L) != 0:
            raise ValueError("oracle_lti_conv rejected its arguments")
        return y


    def scan_fwd_conv(self, xin, conv_w, conv_bias, conv_state_in, delta, delta_bias, delta_softplus, A, B, C,
                      D=None, z=None, h0=None):
        """The Mamba block's main branch from the Conv1D's input (page "Mambaとは？Transformer以外の系列モデル",
        section Mamba blockのarchitecture): x = silu(conv1d(xin) + bias), Δ = delta + delta_bias (softplus
        when asked), then the prefill scan, all in fp64 with nothing rounded between the steps.
        Returns (y, h_final, conv_state_out, x)."""
        x, conv_state_out = self.conv1d(xin, conv_w, conv_bias, conv_state_in, silu=True)
        y, h = self.scan_fwd(x, delta_preprocess(delta, delta_bias, delta_softplus), A, B, C, D, z, h0)
        return y, h, conv_state_out, x

    def scan_step_conv(self, state, conv_state, xin, conv_w, conv_bias, delta, delta_bias, delta_softplus, A, B, C,
                       D=None, z=None):
        """One decode step of that branch: xin, delta, z [b, d]; conv_state [b, d, W-1] (the section
        training、prefill、decodeでは計算の姿が違う keeps it beside the SSM state). Returns (y, new_state,
        new_conv_state, x)."""
        xin = _f64(xin)
        x, new_cs = self.conv1d(xin[:, :, None], conv_w, conv_bias, conv_state, silu=True)
        y, h = self.scan_step(state, x[:, :, 0], delta_preprocess(delta, delta_bias, delta_softplus), A, B, C, D, z)
        return y, h, new_cs, x[:, :, 0]

    def ssd_quadratic(self, x, delta, A, B, C, D=None, z=None, heads=None):
        """y [b, H·P, L] of the scalar-decay SSM in its quadratic form: delta [b, H, L], A [H],
        B, C [b, L, N], D [H·P]; x, z [b, H·P, L]."""
        x = _f64(x)
        delta = _f64(delta)
        if x.ndim != 3 or delta.ndim != 3:
            raise ValueError("x must be [b, H*P, L] and delta [b, H, L]")
        b, d, L = x.shape
        H = delta.shape[1]
        if d % H:
            raise ValueError("channels must split evenly into heads")
        P = d // H
        A = _f64(A, (H,))
        B = _f64(B)
        N = B.shape[2]
        B = _f64(B, (b, L, N))
        C = _f64(C, (b, L, N))
        D = _f64(D, (d,))
        z = _f64(z, (b, d, L))
        y = np.empty_like(x)
        rc = self.lib.oracle_ssd_quadratic(_ptr(x), _ptr(_f64(delta, (b, H, L))), _ptr(A), _ptr(B), _ptr(C),
                                           _ptr(D), _ptr(z), _ptr(y), b, H, P, L, N)
        if rc != 0:
            raise ValueError("oracle_ssd_quadratic rejected its arguments")
        return y


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def zoh(delta, a):
    return default().zoh(delta, a)


def scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None):
    return default().scan_fwd(x, delta, A, B, C, D, z, h0)


def scan_step(state, x, delta, A, B, C, D=None, z=None):
    return default().scan_step(state, x, delta, A, B, C, D, z)


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_final=None):
    return default().scan_bwd(x, delta, A, B, C, D, z, h0, dy, dh_final)


def conv1d(xin, w, bias=None, state=None, silu=True):
    return default().conv1d(xin, w, bias, state, silu)


def lti_kernel(delta, A, B, C, L):
    return default().lti_kernel(delta, A, B, C, L)


def lti_conv(x, K, D=None, z=None):
    return default().lti_conv(x, K, D, z)


def ssd_quadratic(x, delta, A, B, C, D=None, z=None):
    return default().ssd_quadratic(x, delta, A, B, C, D, z)


# ---------------------------------------------------------------------------------------------
# The fused front end of the Mamba block's main branch (page "Mambaとは？Transformer以外の系列モデル",
# section Mamba blockのarchitecture: a causal Conv1D, SiLU, then the selective SSM; section hardware-awareとは
# memory trafficまで設計すること: the parameters are prepared inside the scan's kernel). Written as the
# composition of the pieces above, in fp64: nothing is rounded between the Conv1D and the scan.
# ---------------------------------------------------------------------------------------------
def softplus(v):
    """log(1 + e^v) in fp64, by numpy's logaddexp(0, v) (no overflow for large v). The pages do not give
    Δ's preprocessing; softplus of Δ plus a per-channel bias is the option the library offers."""
    return np.logaddexp(0.0, np.asarray(v, dtype=np.float64))


def delta_preprocess(delta, delta_bias=None, delta_softplus=False):
    """Δ = delta + bias[d] (bias broadcast over b and t), through softplus when asked."""
    dl = _f64(delta)
    if delta_bias is not None:
        shape = (1, -1, 1) if dl.ndim == 3 else (1, -1)
        dl = dl + _f64(delta_bias).reshape(shape)
    return softplus(dl) if delta_softplus else dl


def scan_fwd_conv(xin, conv_w, conv_bias, conv_state_in, delta, delta_bias, delta_softplus, A, B, C, D=None, z=None,
                  h0=None):
    return default().scan_fwd_conv(xin, conv_w, conv_bias, conv_state_in, delta, delta_bias, delta_softplus, A, B, C,
                                   D, z, h0)


def scan_step_conv(state, conv_state, xin, conv_w, conv_bias, delta, delta_bias, delta_softplus, A, B, C, D=None,
                   z=None):
    return default().scan_step_conv(state, conv_state, xin, conv_w, conv_bias, delta, delta_bias, delta_softplus, A, B,
                                    C, D, z)
