"""ctypes binding of libssscan.so: argument checks and marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssscan.so")

SS_OK = 0
SS_F32 = 0
SS_BF16 = 1
MAX_STATE_DIM = 64

_lib = None


class ScanArgs(ctypes.Structure):
    """ss_scan_args of ss_scan.h (same field order and types)."""
    _fields_ = [("batch", ctypes.c_int64), ("channels", ctypes.c_int64), ("state_dim", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("x", ctypes.c_void_p),
                ("dt", ctypes.c_void_p), ("z", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("h0", ctypes.c_void_p), ("reset", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
                ("y", ctypes.c_void_p), ("h_last", ctypes.c_void_p)]


class UpdateArgs(ctypes.Structure):
    """ss_update_args of ss_scan.h (same field order and types)."""
    _fields_ = [("batch", ctypes.c_int64), ("channels", ctypes.c_int64), ("state_dim", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("state", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("dt", ctypes.c_void_p), ("z", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("dt_softplus", ctypes.c_int32), ("y", ctypes.c_void_p)]


class SSError(RuntimeError):
    """A non-zero ss_status returned by the library."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)} (status {code})")


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libssscan.so (built by ``python -m selective_state_space_ss_amd.build``).
    There is no fallback: a missing library raises."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m selective_state_space_ss_amd.build` "
            "(the selective scan has no implementation other than the HIP library)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.ss_scan_fwd.restype = i32
    lib.ss_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), vp]
    lib.ss_scan_fwd_conv.restype = i32
    lib.ss_scan_fwd_conv.argtypes = [ctypes.POINTER(ScanArgs), vp, vp, i64, vp]
    lib.ss_scan_fwd_states.restype = i32
    lib.ss_scan_fwd_states.argtypes = [ctypes.POINTER(ScanArgs), vp, i64, vp]
    lib.ss_gated_scan.restype = i32
    lib.ss_gated_scan.argtypes = [i64, i64, i64, i64, i32, i32] + [vp] * 7 + [vp]
    lib.ss_effective_attention.restype = i32
    lib.ss_effective_attention.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.ss_conv1d_silu.restype = i32
    lib.ss_conv1d_silu.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.ss_dt_proj.restype = i32
    lib.ss_dt_proj.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, i32, vp, vp]
    lib.ss_state_update.restype = i32
    lib.ss_state_update.argtypes = [ctypes.POINTER(UpdateArgs), vp]
    lib.ss_scan_fwd_timed.restype = i32
    lib.ss_scan_fwd_timed.argtypes = [ctypes.POINTER(ScanArgs), vp, vp, vp]
    lib.ss_state_update_timed.restype = i32
    lib.ss_state_update_timed.argtypes = [ctypes.POINTER(UpdateArgs), vp, vp, vp]
    lib.ss_status_str.restype = ctypes.c_char_p
    lib.ss_status_str.argtypes = [i32]
    lib.ss_abi_version.restype = i32
    lib.ss_abi_version.argtypes = []
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().ss_status_str(int(code)).decode()


def abi_version() -> int:
    return load_library().ss_abi_version()


def _io_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return SS_F32
    if dtype == torch.bfloat16:
        return SS_BF16
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {dtype}")


def _check(t, name: str, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(device, stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def ss_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, reset=None, dt_softplus: bool = True,
                *, y=None, h_last=None, return_last_state: bool = True, stream=None, timing_events=None) -> Tuple:
    """Prompt scan on the GPU.

    x, dt, z: [batch, channels, seq]; B, C: [batch, state_dim, seq] (float32 or
    bfloat16, one dtype for all); A: [channels, state_dim]; D, dt_bias:
    [channels]; h0: [batch, channels, state_dim]; reset: [batch, seq] uint8 or
    bool (nonzero = first token of a document). A, D, dt_bias and h0 are
    float32. Returns (y, h_last); h_last is None when return_last_state is
    False. Preallocated outputs may be passed as y= and h_last= (h_last may be
    h0 itself). Runs on the current torch stream unless stream= is given.
    timing_events=(start, stop), raw hipEvent_t handles, calls
    ss_scan_fwd_timed: the kernel's dispatch records them.
    """
    y, h_last, args, dev = _scan_args(x, dt, A, B, C, D, z, dt_bias, h0, reset, dt_softplus, y, h_last,
                                      return_last_state)
    lib = load_library()
    if timing_events is None:
        rc = lib.ss_scan_fwd(ctypes.byref(args), _stream_handle(dev, stream))
    else:
        rc = lib.ss_scan_fwd_timed(ctypes.byref(args), _stream_handle(dev, stream), *timing_events)
    if rc != SS_OK:
        raise SSError(rc, "ss_scan_fwd")
    return y, h_last


def ss_scan_fwd_conv(x_pre, dt, A, B, C, conv_w, conv_b=None, D=None, z=None, dt_bias=None, h0=None, reset=None,
                     dt_softplus: bool = True, *, y=None, h_last=None, return_last_state: bool = True,
                     stream=None) -> Tuple:
    """The prompt scan with its x made in the same kernel from x_pre by the
    causal conv1d + SiLU (x never written to memory): conv_w [channels,
    width] and conv_b [channels] float32, width <= 8; x_pre in place of x,
    every other argument as ss_scan_fwd. Returns (y, h_last)."""
    import torch
    y, h_last, args, dev = _scan_args(x_pre, dt, A, B, C, D, z, dt_bias, h0, reset, dt_softplus, y, h_last,
                                      return_last_state)
    channels = x_pre.shape[1]
    if conv_w.dim() != 2 or conv_w.shape[0] != channels:
        raise ValueError("conv_w must be [channels, width]")
    _check(conv_w, "conv_w", (channels, conv_w.shape[1]), torch.float32, dev)
    if conv_b is not None:
        _check(conv_b, "conv_b", (channels,), torch.float32, dev)
    rc = load_library().ss_scan_fwd_conv(ctypes.byref(args), _ptr(conv_w), _ptr(conv_b), conv_w.shape[1],
                                         _stream_handle(dev, stream))
    if rc != SS_OK:
        raise SSError(rc, "ss_scan_fwd_conv")
    return y, h_last


def ss_scan_fwd_states(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, reset=None,
                       dt_softplus: bool = True, *, time_step: Optional[int] = None, y=None, h_last=None,
                       states=None, stream=None) -> Tuple:
    """The prompt scan that also returns states: (y, h_last, states), with
    states [batch, channels, state_dim, seq] (the state after every token, seq
    fastest like x and y) when time_step is None, else [batch, channels,
    state_dim] (the state after token time_step). Arguments as ss_scan_fwd;
    states= takes a preallocated float32 output."""
    import torch
    y, h_last, args, dev = _scan_args(x, dt, A, B, C, D, z, dt_bias, h0, reset, dt_softplus, y, h_last, True)
    batch, channels, L = x.shape
    N = A.shape[1]
    ts = -1 if time_step is None else int(time_step)
    if time_step is not None and ts < 0:
        raise ValueError("time_step must be None or in [0, seq)")
    shape = (batch, channels, N, L) if ts < 0 else (batch, channels, N)
    if states is None:
        states = torch.empty(shape, dtype=torch.float32, device=dev)
    else:
        _check(states, "states", shape, torch.float32, dev)
    rc = load_library().ss_scan_fwd_states(ctypes.byref(args), _ptr(states), ts, _stream_handle(dev, stream))
    if rc != SS_OK:
        raise SSError(rc, "ss_scan_fwd_states")
    return y, h_last, states


def _scan_args(x, dt, A, B, C, D, z, dt_bias, h0, reset, dt_softplus, y, h_last, return_last_state):
    """Check the scan's tensors, allocate missing outputs; returns y, h_last,
    the ss_scan_args struct, and the device."""
    import torch
    if x.dim() != 3:
        raise ValueError("x must be [batch, channels, seq]")
    batch, channels, L = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ss_scan_fwd runs on the GPU: x must be a device tensor")
    io = x.dtype
    code = _io_code(io)
    if A.dim() != 2 or A.shape[0] != channels:
        raise ValueError("A must be [channels, state_dim]")
    N = A.shape[1]
    _check(x, "x", (batch, channels, L), io, dev)
    _check(dt, "dt", (batch, channels, L), io, dev)
    _check(A, "A", (channels, N), torch.float32, dev)
    _check(B, "B", (batch, N, L), io, dev)
    _check(C, "C", (batch, N, L), io, dev)
    if D is not None:
        _check(D, "D", (channels,), torch.float32, dev)
    if z is not None:
        _check(z, "z", (batch, channels, L), io, dev)
    if dt_bias is not None:
        _check(dt_bias, "dt_bias", (channels,), torch.float32, dev)
    if h0 is not None:
        _check(h0, "h0", (batch, channels, N), torch.float32, dev)
    if reset is not None:
        if reset.dtype == torch.bool:
            reset = reset.view(torch.uint8)
        _check(reset, "reset", (batch, L), torch.uint8, dev)
    if y is None:
        y = torch.empty((batch, channels, L), dtype=io, device=dev)
    else:
        _check(y, "y", (batch, channels, L), io, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((batch, channels, N), dtype=torch.float32, device=dev)
    elif h_last is not None:
        _check(h_last, "h_last", (batch, channels, N), torch.float32, dev)
    args = ScanArgs(batch=batch, channels=channels, state_dim=N, seqlen=L, io_dtype=code, x=_ptr(x), dt=_ptr(dt),
                    z=_ptr(z), B=_ptr(B), C=_ptr(C), A=_ptr(A), D=_ptr(D), dt_bias=_ptr(dt_bias), h0=_ptr(h0),
                    reset=_ptr(reset), dt_softplus=int(bool(dt_softplus)), y=_ptr(y), h_last=_ptr(h_last))
    return y, h_last, args, dev




def ss_gated_scan(q, k, v, gamma, s0=None, *, state_dtype=None, y=None, final_state=None,
                  return_final_state: bool = True, stream=None) -> Tuple:
    """Scalar-gated state scan on the GPU: S_t = gamma_t S_{t-1} + k_t v_t^T,
    y_t = q_t^T S_t, in fp32. q, k: [batch, seq, dk]; v: [batch, seq, dv]
    (float32 or bfloat16, one dtype); gamma: [batch, seq] float32; s0:
    [batch, dk, dv] in state_dtype, or None (zeros). state_dtype defaults to
    that of s0 (or of a given final_state), else to q's dtype, as the page
    returns the final state; float32 keeps a state carried across calls
    unrounded. Returns (y [batch, seq, dv] in q's dtype,
    final_state [batch, dk, dv] in state_dtype, or None when
    return_final_state is False). Strided inputs are copied to contiguous ones
    first (the library takes contiguous arrays); preallocated outputs may be
    passed as y= and final_state= (final_state may be s0 itself)."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [batch, seq, dk] and v [batch, seq, dv]")
    batch, L, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("ss_gated_scan runs on the GPU: q must be a device tensor")
    io = q.dtype
    code = _io_code(io)
    if state_dtype is not None:
        sdt = state_dtype
    elif s0 is not None:
        sdt = s0.dtype
    elif final_state is not None:
        sdt = final_state.dtype
    else:
        sdt = io
    scode = _io_code(sdt)
    q, k, v, gamma = q.contiguous(), k.contiguous(), v.contiguous(), gamma.contiguous()
    _check(q, "q", (batch, L, dk), io, dev)
    _check(k, "k", (batch, L, dk), io, dev)
    _check(v, "v", (batch, L, dv), io, dev)
    _check(gamma, "gamma", (batch, L), torch.float32, dev)
    if s0 is not None:
        _check(s0, "s0", (batch, dk, dv), sdt, dev)
    if y is None:
        y = torch.empty((batch, L, dv), dtype=io, device=dev)
    else:
        _check(y, "y", (batch, L, dv), io, dev)
    if return_final_state and final_state is None:
        final_state = torch.empty((batch, dk, dv), dtype=sdt, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", (batch, dk, dv), sdt, dev)
    rc = load_library().ss_gated_scan(batch, L, dk, dv, code, scode, _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(s0),
                                      _ptr(y), _ptr(final_state), _stream_handle(dev, stream))
    if rc != SS_OK:
        raise SSError(rc, "ss_gated_scan")
    return y, final_state


def ss_effective_attention(dt, A, B, C, dt_bias=None, *, dt_softplus: bool = True,
                           include_dt_scaling: bool = False, per_state_coord: bool = False, out=None,
                           stream=None):
    """Effective attention of the selective scan on the GPU:
    M[b, c, i, j] = sum_n C[b, n, i] prod_{k=j+1..i} exp(A[c, n] dt[b, c, k]) B[b, n, j]
    for j <= i, 0 above the diagonal, with dt the scan's step size
    (softplus(dt + dt_bias) unless dt_softplus is False). dt: [batch,
    channels, seq]; B, C: [batch, state_dim, seq] (float32 or bfloat16, one
    dtype); A: [channels, state_dim] float32; dt_bias: [channels] float32 or
    None. include_dt_scaling multiplies column j by dt_j (then y = M x + D x
    before the gate); per_state_coord keeps the state coordinate axis.
    Returns float32 [batch, channels, seq, seq] or [batch, channels,
    state_dim, seq, seq] (written into `out` when given)."""
    import torch
    if dt.dim() != 3 or A.dim() != 2:
        raise ValueError("dt must be [batch, channels, seq] and A [channels, state_dim]")
    batch, channels, L = dt.shape
    N = A.shape[1]
    dev = dt.device
    if dev.type != "cuda":
        raise ValueError("ss_effective_attention runs on the GPU: dt must be a device tensor")
    io = dt.dtype
    code = _io_code(io)
    dt, A, B, C = dt.contiguous(), A.contiguous(), B.contiguous(), C.contiguous()
    _check(A, "A", (channels, N), torch.float32, dev)
    _check(B, "B", (batch, N, L), io, dev)
    _check(C, "C", (batch, N, L), io, dev)
    if dt_bias is not None:
        dt_bias = dt_bias.contiguous()
        _check(dt_bias, "dt_bias", (channels,), torch.float32, dev)
    shape = (batch, channels, N, L, L) if per_state_coord else (batch, channels, L, L)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    else:
        _check(out, "out", shape, torch.float32, dev)
    rc = load_library().ss_effective_attention(batch, channels, N, L, code, _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                               _ptr(dt_bias), int(bool(dt_softplus)),
                                               int(bool(include_dt_scaling)), int(bool(per_state_coord)),
                                               _ptr(out), _stream_handle(dev, stream))
    if rc != SS_OK:
        raise SSError(rc, "ss_effective_attention")
    return out


def ss_conv1d_silu(x_pre, conv_w, conv_b=None, reset=None, *, out=None, stream=None):
    """x = silu(causal depthwise conv1d of x_pre + conv_b) on the GPU.
    x_pre: [batch, channels, seq] float32 or bfloat16; conv_w: [channels,
    width] float32 (width <= 8; conv_w[:, -1] meets the current token);
    conv_b: [channels] float32 or None; reset: [batch, seq] bool/uint8 or
    None (a document's taps stop at its first token). Returns x like x_pre."""
    import torch
    if x_pre.dim() != 3 or conv_w.dim() != 2:
        raise ValueError("x_pre must be [batch, channels, seq] and conv_w [channels, width]")
    batch, channels, L = x_pre.shape
    dev = x_pre.device
    if dev.type != "cuda":
        raise ValueError("ss_conv1d_silu runs on the GPU: x_pre must be a device tensor")
    io = x_pre.dtype
    code = _io_code(io)
    x_pre, conv_w = x_pre.contiguous(), conv_w.contiguous()
    _check(conv_w, "conv_w", (channels, conv_w.shape[1]), torch.float32, dev)
    if conv_b is not None:
        conv_b = conv_b.contiguous()
        _check(conv_b, "conv_b", (channels,), torch.float32, dev)
    if reset is not None:
        reset = reset.to(torch.uint8).contiguous()
        _check(reset, "reset", (batch, L), torch.uint8, dev)
    if out is None:
        out = torch.empty_like(x_pre)
    else:
        _check(out, "out", (batch, channels, L), io, dev)
    rc = load_library().ss_conv1d_silu(batch, channels, L, conv_w.shape[1], code, _ptr(x_pre), _ptr(conv_w),
                                       _ptr(conv_b), _ptr(reset), _ptr(out), _stream_handle(dev, stream))
    if rc != SS_OK:
        raise SSError(rc, "ss_conv1d_silu")
    return out


def ss_dt_proj(w_dt, delta, dt_bias=None, *, apply_softplus: bool = False, out=None, stream=None):
    """dt[b, c, t] = sum_k w_dt[c, k] delta[b, t, k] on the GPU's matrix cores
    (fp32 accumulation), optionally softplus(dt + dt_bias[c]). w_dt:
    [channels, rank]; delta: [batch, seq, rank] (token-major), one dtype
    (float32 or bfloat16); dt_bias: [channels] float32 or None. Returns dt
    [batch, channels, seq] in that dtype."""
    import torch
    if w_dt.dim() != 2 or delta.dim() != 3:
        raise ValueError("w_dt must be [channels, rank] and delta [batch, seq, rank]")
    channels, R = w_dt.shape
    batch, L = delta.shape[:2]
    dev = delta.device
    if dev.type != "cuda":
        raise ValueError("ss_dt_proj runs on the GPU: delta must be a device tensor")
    io = delta.dtype
    code = _io_code(io)
    w_dt, delta = w_dt.contiguous(), delta.contiguous()
    _check(w_dt, "w_dt", (channels, R), io, dev)
    _check(delta, "delta", (batch, L, R), io, dev)
    if dt_bias is not None:
        dt_bias = dt_bias.contiguous()
        _check(dt_bias, "dt_bias", (channels,), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, channels, L), dtype=io, device=dev)
    else:
        _check(out, "out", (batch, channels, L), io, dev)
    rc = load_library().ss_dt_proj(batch, channels, L, R, code, _ptr(w_dt), _ptr(delta), _ptr(dt_bias),
                                   int(bool(apply_softplus)), _ptr(out), _stream_handle(dev, stream))
    if rc != SS_OK:
        raise SSError(rc, "ss_dt_proj")
    return out


def ss_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus: bool = True, *, y=None,
                    stream=None, timing_events=None):
    """Single-token decode step on the GPU; `state` ([batch, channels,
    state_dim] float32) is updated in place. x, dt, z: [batch, channels];
    B, C: [batch, state_dim]. Returns y [batch, channels].
    timing_events=(start, stop), raw hipEvent_t handles, calls
    ss_state_update_timed: the kernel's dispatch records them."""
    import torch
    if state.dim() != 3:
        raise ValueError("state must be [batch, channels, state_dim]")
    batch, channels, N = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("ss_state_update runs on the GPU: state must be a device tensor")
    io = x.dtype
    code = _io_code(io)
    _check(state, "state", (batch, channels, N), torch.float32, dev)
    _check(x, "x", (batch, channels), io, dev)
    _check(dt, "dt", (batch, channels), io, dev)
    _check(A, "A", (channels, N), torch.float32, dev)
    _check(B, "B", (batch, N), io, dev)
    _check(C, "C", (batch, N), io, dev)
    if D is not None:
        _check(D, "D", (channels,), torch.float32, dev)
    if z is not None:
        _check(z, "z", (batch, channels), io, dev)
    if dt_bias is not None:
        _check(dt_bias, "dt_bias", (channels,), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, channels), dtype=io, device=dev)
    else:
        _check(y, "y", (batch, channels), io, dev)
    lib = load_library()
    args = UpdateArgs(batch=batch, channels=channels, state_dim=N, io_dtype=code, state=_ptr(state), x=_ptr(x),
                      dt=_ptr(dt), z=_ptr(z), B=_ptr(B), C=_ptr(C), A=_ptr(A), D=_ptr(D), dt_bias=_ptr(dt_bias),
                      dt_softplus=int(bool(dt_softplus)), y=_ptr(y))
    if timing_events is None:
        rc = lib.ss_state_update(ctypes.byref(args), _stream_handle(dev, stream))
    else:
        rc = lib.ss_state_update_timed(ctypes.byref(args), _stream_handle(dev, stream), *timing_events)
    if rc != SS_OK:
        raise SSError(rc, "ss_state_update")
    return y
