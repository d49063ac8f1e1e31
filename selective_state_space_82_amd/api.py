"""Thin Python binding of libssmscan.so: torch tensors in, raw device pointers to the C ABI out.

Argument marshalling only: every step of the scan runs in the library's HIP kernels. torch
provides device memory and the current stream. There is no fallback: if the library is missing
or the tensors are not on a ROCm GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_OK = 0
STATUS_NAMES = {0: "SSM_OK", 1: "SSM_ERR_NULL", 2: "SSM_ERR_SHAPE", 3: "SSM_ERR_UNSUPPORTED",
                4: "SSM_ERR_HIP", 5: "SSM_ERR_ALIAS", 6: "SSM_ERR_SCRATCH"}
SSM_ERR_SCRATCH = 6
NOALLOC_SCRATCH_BYTES = 32 << 20


class SsmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class FwdOpts(ctypes.Structure):
    """ssm_fwd_opts_t."""
    _fields_ = [("seg_len", ctypes.c_int32), ("lanes_per_channel", ctypes.c_int32),
                ("initial_state", ctypes.c_void_p), ("ev_begin", ctypes.c_void_p),
                ("ev_end", ctypes.c_void_p), ("reserved", ctypes.c_int64 * 4)]


class FwdPlan(ctypes.Structure):
    """ssm_fwd_plan_t."""
    _fields_ = [("seg_len", ctypes.c_int32), ("lanes_per_channel", ctypes.c_int32),
                ("states_per_lane", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("waves_per_segment", ctypes.c_int64),
                ("groups_output_pass", ctypes.c_int64), ("groups_aggregate_pass", ctypes.c_int64),
                ("scratch_bytes", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library with argument types declared (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    fwd = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    L.ssm_scan_fwd.argtypes = fwd
    L.ssm_scan_fwd.restype = i32
    L.ssm_scan_fwd_ex.argtypes = fwd + [ctypes.POINTER(FwdOpts)]
    L.ssm_scan_fwd_ex.restype = i32
    L.ssm_scan_fwd_noalloc.argtypes = fwd + [ctypes.POINTER(FwdOpts)]
    L.ssm_scan_fwd_noalloc.restype = i32
    L.ssm_scan_fwd_plan.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(FwdOpts), ctypes.POINTER(FwdPlan)]
    L.ssm_scan_fwd_plan.restype = i32
    L.ssm_scan_step.argtypes = [vp] * 9 + [i64, i64, i64, i32, vp]
    L.ssm_scan_step.restype = i32
    L.ssm_scan_bwd.argtypes = [vp] * 18 + [i64, i64, i64, i64, i32, vp]
    L.ssm_scan_bwd.restype = i32
    L.ssm_conv1d_fwd.argtypes = [vp] * 6 + [i64, i64, i64, i64, i32, i32, vp]
    L.ssm_conv1d_fwd.restype = i32
    L.ssm_conv1d_step.argtypes = [vp] * 5 + [i64, i64, i64, i32, i32, vp]
    L.ssm_conv1d_step.restype = i32
    L.ssm_scan_fwd_conv.argtypes = [vp, vp, vp, vp, i64, vp, vp, i32] + [vp] * 10 + [i64, i64, i64, i64, i32, vp]
    L.ssm_scan_fwd_conv.restype = i32
    L.ssm_scan_step_conv.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, i32] + [vp] * 7 + [i64, i64, i64, i32, vp]
    L.ssm_scan_step_conv.restype = i32
    L.ssm_lti_kernel.argtypes = [vp] * 5 + [i64, i64, i64, vp]
    L.ssm_lti_kernel.restype = i32
    L.ssm_lti_conv.argtypes = [vp] * 5 + [i64, i64, i64, i32, vp]
    L.ssm_lti_conv.restype = i32
    L.ssm_lti_fwd.argtypes = [vp] * 8 + [i64, i64, i64, i64, i32, vp]
    L.ssm_lti_fwd.restype = i32
    L.ssm_ssd_fwd.argtypes = [vp] * 10 + [i64, i64, i64, i64, i64, i32, vp]
    L.ssm_ssd_fwd.restype = i32
    L.ssm_status_string.argtypes = [i32]
    L.ssm_status_string.restype = ctypes.c_char_p
    L.ssm_abi_version.argtypes = []
    L.ssm_abi_version.restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().ssm_status_string(int(status)).decode()


def _raise(status: int, what: str):
    if status != SSM_OK:
        raise SsmError(status, f"{what}: {status_string(status)}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SSM_F32
    if t == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported storage dtype {t}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def ssm_scan_fwd(x, delta, A, B, C, D=None, z=None, *, y=None, final_state=None, return_final_state=True,
                 seg_len=0, lanes_per_channel=0, initial_state=None, events=None, noalloc=False):
    """Prefill scan. x, delta, z: [b, d, L]; A: [d, N] fp32; B, C: [b, L, N]; D: [d] fp32.
    x, delta, z, B, C share one storage dtype (float32 or bfloat16); y gets it too.
    Returns (y, final_state) (final_state is None when return_final_state is False and none is given).
    events: optional (begin, end) torch.cuda.Event pair recorded around the output-pass kernel.
    noalloc: call ssm_scan_fwd_noalloc (scratch in the library's fixed device array; y and final_state
    should then be given, since allocating them here would defeat the purpose)."""
    if x.dim() != 3:
        raise ValueError("x must be [b, d, L]")
    b, d, L = x.shape
    if A.dim() != 2:
        raise ValueError("A must be [d, N]")
    N = A.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a ROCm GPU")
    st = x.dtype
    code = _dtype_code(st)
    _check("delta", delta, (b, d, L), st, dev)
    _check("A", A, (d, N), torch.float32, dev)
    _check("B", B, (b, L, N), st, dev)
    _check("C", C, (b, L, N), st, dev)
    _check("D", D, (d,), torch.float32, dev)
    _check("z", z, (b, d, L), st, dev)
    _check("x", x, (b, d, L), st, dev)
    _check("initial_state", initial_state, (b, d, N), torch.float32, dev)
    if y is None:
        y = torch.empty((b, d, L), dtype=st, device=dev)
    _check("y", y, (b, d, L), st, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((b, d, N), dtype=torch.float32, device=dev)
    _check("final_state", final_state, (b, d, N), torch.float32, dev)
    args = [_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), _ptr(final_state),
            b, d, L, N, code, _stream(dev)]
    if noalloc or seg_len or lanes_per_channel or initial_state is not None or events is not None:
        o = FwdOpts()
        o.seg_len = int(seg_len)
        o.lanes_per_channel = int(lanes_per_channel)
        o.initial_state = None if initial_state is None else initial_state.data_ptr()
        if events is not None:
            o.ev_begin = events[0].cuda_event
            o.ev_end = events[1].cuda_event
        fn = lib().ssm_scan_fwd_noalloc if noalloc else lib().ssm_scan_fwd_ex
        status = fn(*args, ctypes.byref(o))
    else:
        status = lib().ssm_scan_fwd(*args)
    _raise(status, "ssm_scan_fwd_noalloc" if noalloc else "ssm_scan_fwd")
    return y, final_state


def ssm_scan_fwd_conv(xin, conv_w, delta, A, B, C, D=None, z=None, *, conv_bias=None, conv_state_in=None,
                      delta_bias=None, delta_softplus=False, initial_state=None, y=None, final_state=None,
                      conv_state_out=None, x_out=None, return_states=True, want_x=False):
    """The Mamba block's main branch in one prefill pass: Conv1D (conv_w [d, W], W <= 4) + SiLU on xin
    [b, d, L], Δ = delta + delta_bias (softplus when delta_softplus), then the scan. Returns
    (y, final_state, conv_state_out, x_out); the states are allocated when return_states is set and none is
    given, x_out (the convolved input) when want_x is set."""
    if xin.dim() != 3 or conv_w.dim() != 2:
        raise ValueError("xin must be [b, d, L] and conv_w [d, W]")
    b, d, L = xin.shape
    N = A.shape[1]
    W = conv_w.shape[1]
    dev = xin.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a ROCm GPU")
    st = xin.dtype
    code = _dtype_code(st)
    f32 = torch.float32
    for name, t, shape, dt in (("delta", delta, (b, d, L), st), ("A", A, (d, N), f32), ("B", B, (b, L, N), st),
                               ("C", C, (b, L, N), st), ("D", D, (d,), f32), ("z", z, (b, d, L), st),
                               ("conv_w", conv_w, (d, W), f32), ("conv_bias", conv_bias, (d,), f32),
                               ("conv_state_in", conv_state_in, (b, d, W - 1), f32),
                               ("delta_bias", delta_bias, (d,), f32), ("initial_state", initial_state, (b, d, N), f32),
                               ("xin", xin, (b, d, L), st)):
        _check(name, t, shape, dt, dev)
    if y is None:
        y = torch.empty((b, d, L), dtype=st, device=dev)
    if return_states and final_state is None:
        final_state = torch.empty((b, d, N), dtype=f32, device=dev)
    if return_states and conv_state_out is None and W > 1:
        conv_state_out = torch.empty((b, d, W - 1), dtype=f32, device=dev)
    if want_x and x_out is None:
        x_out = torch.empty((b, d, L), dtype=st, device=dev)
    _check("y", y, (b, d, L), st, dev)
    _check("final_state", final_state, (b, d, N), f32, dev)
    _check("conv_state_out", conv_state_out, (b, d, W - 1), f32, dev)
    _check("x_out", x_out, (b, d, L), st, dev)
    status = lib().ssm_scan_fwd_conv(_ptr(xin), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state_in), W, _ptr(delta),
                                     _ptr(delta_bias), int(bool(delta_softplus)), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                     _ptr(z), _ptr(initial_state), _ptr(y), _ptr(final_state), _ptr(conv_state_out),
                                     _ptr(x_out), b, d, L, N, code, _stream(dev))
    _raise(status, "ssm_scan_fwd_conv")
    return y, final_state, conv_state_out, x_out


def ssm_scan_step_conv(state, conv_state, xin, conv_w, delta, A, B, C, D=None, z=None, *, conv_bias=None,
                       delta_bias=None, delta_softplus=False, y=None, x_out=None):
    """One decode step of the Mamba block's main branch: state [b, d, N] and conv_state [b, d, W-1] (fp32,
    both updated in place); xin, delta, z [b, d]; conv_w [d, W]. Returns (y, x_out) (x_out None unless
    given)."""
    b, d, N = state.shape
    W = conv_w.shape[1]
    dev = state.device
    st = xin.dtype
    code = _dtype_code(st)
    f32 = torch.float32
    for name, t, shape, dt in (("state", state, (b, d, N), f32), ("conv_state", conv_state, (b, d, W - 1), f32),
                               ("xin", xin, (b, d), st), ("delta", delta, (b, d), st), ("A", A, (d, N), f32),
                               ("B", B, (b, N), st), ("C", C, (b, N), st), ("D", D, (d,), f32), ("z", z, (b, d), st),
                               ("conv_w", conv_w, (d, W), f32), ("conv_bias", conv_bias, (d,), f32),
                               ("delta_bias", delta_bias, (d,), f32)):
        _check(name, t, shape, dt, dev)
    if y is None:
        y = torch.empty((b, d), dtype=st, device=dev)
    _check("y", y, (b, d), st, dev)
    _check("x_out", x_out, (b, d), st, dev)
    status = lib().ssm_scan_step_conv(_ptr(state), _ptr(conv_state) if W > 1 else None, _ptr(xin), _ptr(conv_w),
                                      _ptr(conv_bias), W, _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                      _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), _ptr(x_out), b, d, N, code,
                                      _stream(dev))
    _raise(status, "ssm_scan_step_conv")
    return y, x_out


def ssm_scan_step(state, x, delta, A, B, C, D=None, z=None, *, y=None):
    """Decode step: state [b, d, N] fp32 (updated in place); x, delta, z [b, d]; B, C [b, N];
    A [d, N] fp32; D [d] fp32. Returns y [b, d]."""
    if state.dim() != 3:
        raise ValueError("state must be [b, d, N]")
    b, d, N = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a ROCm GPU")
    st = x.dtype
    code = _dtype_code(st)
    _check("state", state, (b, d, N), torch.float32, dev)
    _check("x", x, (b, d), st, dev)
    _check("delta", delta, (b, d), st, dev)
    _check("A", A, (d, N), torch.float32, dev)
    _check("B", B, (b, N), st, dev)
    _check("C", C, (b, N), st, dev)
    _check("D", D, (d,), torch.float32, dev)
    _check("z", z, (b, d), st, dev)
    if y is None:
        y = torch.empty((b, d), dtype=st, device=dev)
    _check("y", y, (b, d), st, dev)
    status = lib().ssm_scan_step(_ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(y), b, d, N, code, _stream(dev))
    _raise(status, "ssm_scan_step")
    return y


def ssm_scan_bwd(x, delta, A, B, C, D=None, z=None, *, dy, initial_state=None, d_final_state=None,
                 want_dD=True, want_d_initial_state=True) -> dict:
    """Gradients of ssm_scan_fwd for an upstream gradient dy [b, d, L] (and optionally d_final_state
    [b, d, N]). Returns a dict: dx, ddelta, dz ([b, d, L], storage dtype; dz None without z),
    dA [d, N], dB, dC [b, L, N], dD [d] (None unless want_dD), d_initial_state [b, d, N] (None unless
    want_d_initial_state), all fp32 except the first three."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [b, d, L] and A [d, N]")
    b, d, L = x.shape
    N = A.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a ROCm GPU")
    st = x.dtype
    code = _dtype_code(st)
    for name, t, shape, dt in (("delta", delta, (b, d, L), st), ("A", A, (d, N), torch.float32),
                               ("B", B, (b, L, N), st), ("C", C, (b, L, N), st), ("D", D, (d,), torch.float32),
                               ("z", z, (b, d, L), st), ("dy", dy, (b, d, L), st),
                               ("initial_state", initial_state, (b, d, N), torch.float32),
                               ("d_final_state", d_final_state, (b, d, N), torch.float32)):
        _check(name, t, shape, dt, dev)
    f32 = torch.float32
    out = {"dx": torch.empty((b, d, L), dtype=st, device=dev), "ddelta": torch.empty((b, d, L), dtype=st, device=dev),
           "dz": None if z is None else torch.empty((b, d, L), dtype=st, device=dev),
           "dA": torch.empty((d, N), dtype=f32, device=dev), "dB": torch.empty((b, L, N), dtype=f32, device=dev),
           "dC": torch.empty((b, L, N), dtype=f32, device=dev),
           "dD": torch.empty((d,), dtype=f32, device=dev) if want_dD else None,
           "d_initial_state": torch.empty((b, d, N), dtype=f32, device=dev) if want_d_initial_state else None}
    status = lib().ssm_scan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(initial_state), _ptr(dy), _ptr(d_final_state), _ptr(out["dx"]),
                                _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                                _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["d_initial_state"]), b, d, L, N, code,
                                _stream(dev))
    _raise(status, "ssm_scan_bwd")
    return out


def ssm_conv1d_fwd(xin, w, bias=None, *, state_in=None, x_out=None, state_out=None, return_state=True,
                   silu=True):
    """Causal depthwise Conv1D (+ SiLU): xin [b, d, L] (float32 or bfloat16), w [d, W] fp32, bias [d] fp32.
    Returns (x [b, d, L] in xin's dtype, state [b, d, W-1] fp32 or None)."""
    if xin.dim() != 3 or w.dim() != 2:
        raise ValueError("xin must be [b, d, L] and w [d, W]")
    b, d, L = xin.shape
    W = w.shape[1]
    dev = xin.device
    st = xin.dtype
    code = _dtype_code(st)
    _check("xin", xin, (b, d, L), st, dev)
    _check("w", w, (d, W), torch.float32, dev)
    _check("bias", bias, (d,), torch.float32, dev)
    _check("state_in", state_in, (b, d, W - 1), torch.float32, dev)
    if x_out is None:
        x_out = torch.empty((b, d, L), dtype=st, device=dev)
    _check("x_out", x_out, (b, d, L), st, dev)
    if state_out is None and return_state and W > 1:
        state_out = torch.empty((b, d, W - 1), dtype=torch.float32, device=dev)
    _check("state_out", state_out, (b, d, W - 1), torch.float32, dev)
    status = lib().ssm_conv1d_fwd(_ptr(xin), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(x_out), _ptr(state_out),
                                  b, d, L, W, int(bool(silu)), code, _stream(dev))
    _raise(status, "ssm_conv1d_fwd")
    return x_out, state_out


def ssm_lti_kernel(delta, A, B, C, L, *, K=None):
    """K̄ [d, L] fp32 of the time-invariant system per channel: delta [d], A, B, C [d, N], all fp32."""
    if A.dim() != 2:
        raise ValueError("A must be [d, N]")
    d, N = A.shape
    dev = A.device
    for name, t, shape in (("delta", delta, (d,)), ("A", A, (d, N)), ("B", B, (d, N)), ("C", C, (d, N))):
        _check(name, t, shape, torch.float32, dev)
    if K is None:
        K = torch.empty((d, int(L)), dtype=torch.float32, device=dev)
    _check("K", K, (d, int(L)), torch.float32, dev)
    status = lib().ssm_lti_kernel(_ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(K), d, int(L), N, _stream(dev))
    _raise(status, "ssm_lti_kernel")
    return K


def ssm_lti_conv(x, K, D=None, z=None, *, y=None):
    """y = x ∗ K̄ + D·x (· silu(z)) by FFT: x, z [b, d, L] (float32 or bfloat16), K [d, L] fp32, D [d] fp32."""
    if x.dim() != 3:
        raise ValueError("x must be [b, d, L]")
    b, d, L = x.shape
    dev, st = x.device, x.dtype
    code = _dtype_code(st)
    _check("K", K, (d, L), torch.float32, dev)
    _check("D", D, (d,), torch.float32, dev)
    _check("z", z, (b, d, L), st, dev)
    if y is None:
        y = torch.empty((b, d, L), dtype=st, device=dev)
    _check("y", y, (b, d, L), st, dev)
    status = lib().ssm_lti_conv(_ptr(x), _ptr(K), _ptr(D), _ptr(z), _ptr(y), b, d, L, code, _stream(dev))
    _raise(status, "ssm_lti_conv")
    return y


def ssm_lti_fwd(x, delta, A, B, C, D=None, z=None, *, y=None):
    """The LTI scan as a convolution in one call: K̄ from (delta [d], A, B, C [d, N]), then ssm_lti_conv."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [b, d, L] and A [d, N]")
    b, d, L = x.shape
    N = A.shape[1]
    dev, st = x.device, x.dtype
    code = _dtype_code(st)
    for name, t, shape in (("delta", delta, (d,)), ("A", A, (d, N)), ("B", B, (d, N)), ("C", C, (d, N)),
                           ("D", D, (d,))):
        _check(name, t, shape, torch.float32, dev)
    _check("z", z, (b, d, L), st, dev)
    if y is None:
        y = torch.empty((b, d, L), dtype=st, device=dev)
    _check("y", y, (b, d, L), st, dev)
    status = lib().ssm_lti_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                               b, d, L, N, code, _stream(dev))
    _raise(status, "ssm_lti_fwd")
    return y


def ssm_ssd_fwd(x, delta, A, B, C, D=None, z=None, *, y=None, initial_state=None, final_state=None,
                return_final_state=True):
    """Scalar-decay (state space duality) form, chunked on the MFMA units. x, z: [b, H*P, L] with P = 64;
    delta: [b, H, L]; A: [H] fp32 (one decay per head); B, C: [b, L, N] with N in {32, 64, 128};
    D: [H*P] fp32. Returns (y, final_state [b, H*P, N] fp32 or None)."""
    if x.dim() != 3 or delta.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [b, H*P, L], delta [b, H, L], B and C [b, L, N]")
    b, d, L = x.shape
    H = delta.shape[1]
    if d % H:
        raise ValueError("the channels must split evenly into heads")
    P, N = d // H, B.shape[2]
    dev, st = x.device, x.dtype
    code = _dtype_code(st)
    _check("delta", delta, (b, H, L), st, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("B", B, (b, L, N), st, dev)
    _check("C", C, (b, L, N), st, dev)
    _check("D", D, (d,), torch.float32, dev)
    _check("z", z, (b, d, L), st, dev)
    _check("initial_state", initial_state, (b, d, N), torch.float32, dev)
    if y is None:
        y = torch.empty((b, d, L), dtype=st, device=dev)
    _check("y", y, (b, d, L), st, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((b, d, N), dtype=torch.float32, device=dev)
    _check("final_state", final_state, (b, d, N), torch.float32, dev)
    status = lib().ssm_ssd_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(initial_state), _ptr(y), _ptr(final_state), b, H, P, L, N, code, _stream(dev))
    _raise(status, "ssm_ssd_fwd")
    return y, final_state


def ssm_conv1d_step(state, xin, w, bias=None, *, x_out=None, silu=True):
    """Decode step of the Conv1D: state [b, d, W-1] fp32 (shifted in place), xin [b, d]. Returns x [b, d]."""
    b, d = xin.shape
    W = w.shape[1]
    dev = xin.device
    st = xin.dtype
    code = _dtype_code(st)
    _check("state", state, (b, d, W - 1), torch.float32, dev)
    _check("w", w, (d, W), torch.float32, dev)
    _check("bias", bias, (d,), torch.float32, dev)
    if x_out is None:
        x_out = torch.empty((b, d), dtype=st, device=dev)
    _check("x_out", x_out, (b, d), st, dev)
    status = lib().ssm_conv1d_step(_ptr(state), _ptr(xin), _ptr(w), _ptr(bias), _ptr(x_out), b, d, W,
                                   int(bool(silu)), code, _stream(dev))
    _raise(status, "ssm_conv1d_step")
    return x_out


def ssm_scan_fwd_plan(b, d, L, N, dtype=torch.float32, seg_len=0, lanes_per_channel=0) -> dict:
    """The launch plan ssm_scan_fwd would use (host only)."""
    o = FwdOpts()
    o.seg_len = int(seg_len)
    o.lanes_per_channel = int(lanes_per_channel)
    p = FwdPlan()
    status = lib().ssm_scan_fwd_plan(b, d, L, N, _dtype_code(dtype), ctypes.byref(o), ctypes.byref(p))
    _raise(status, "ssm_scan_fwd_plan")
    return {k: getattr(p, k) for k, _ in FwdPlan._fields_}
