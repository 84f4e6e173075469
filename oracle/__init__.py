"""CPU oracle of the Mamba-1 S6 selective scan (fp64, sequential token loop).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may call this package; the product path
(the HIP library and its binding) never imports it, and it imports nothing
from there.

The arithmetic lives in ``ss_oracle.c`` (plain C, IEEE double, libm); this
module only marshals numpy arrays into it and splits independent (batch,
channel) rows over threads (ctypes releases the GIL during each call). Rows
never interact, so the split changes no result: every row's token loop stays
sequential in one call.

Every function here is pinned: the scan and the decode step by
``tests/test_oracle_pins.py``, the scalar-gated scan by
``tests/test_oracle_gated_pins.py``, the effective attention by
``tests/test_oracle_attention_pins.py``, the conv1d + SiLU and dt_proj
producers by ``tests/test_oracle_producer_pins.py``; ``tests/test_oracle_mutants.py``
checks that the pins catch planted mistakes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_LIB = os.path.join(_HERE, "libssoracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile ss_oracle.c with gcc (no fast-math) into libssoracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_scan.argtypes = [i64, i64, i64, i64] + [dp] * 10 + [ctypes.c_int] + [dp] * 3 + [i64, i64]
        lib.oracle_update.restype = ctypes.c_int
        lib.oracle_update.argtypes = [i64, i64, i64] + [dp] * 9 + [ctypes.c_int, dp, i64, i64]
        lib.oracle_gated_scan.restype = ctypes.c_int
        lib.oracle_gated_scan.argtypes = [i64, i64, i64, i64] + [dp] * 7 + [i64, i64]
        lib.oracle_effective_attention.restype = ctypes.c_int
        lib.oracle_effective_attention.argtypes = [i64, i64, i64, i64] + [dp] * 5 + [ctypes.c_int] * 3 + [
            dp, i64, i64]
        lib.oracle_conv1d_silu.restype = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [i64, i64, i64, i64] + [dp] * 5 + [i64, i64]
        lib.oracle_dt_proj.restype = ctypes.c_int
        lib.oracle_dt_proj.argtypes = [i64, i64, i64, i64] + [dp] * 3 + [ctypes.c_int, dp, i64, i64]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        _lib = lib
    return _lib


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


MAX_DEFAULT_THREADS = 16   # a one-GPU share of the host's cores


def _threads(threads: Optional[int]) -> int:
    if threads is not None:
        return max(1, int(threads))
    return max(1, min(MAX_DEFAULT_THREADS, len(os.sched_getaffinity(0))))


def _split_rows(rows: int, parts: int):
    parts = max(1, min(parts, rows))
    edges = [rows * k // parts for k in range(parts + 1)]
    return [(edges[k], edges[k + 1]) for k in range(parts) if edges[k + 1] > edges[k]]


def softplus(v: float) -> float:
    return _load().oracle_softplus(float(v))


def scan(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, reset=None, dt_softplus=True,
         return_states=False, threads=None):
    """Prompt scan. x, dt, z: [batch, channels, L]; B, C: [batch, N, L];
    A: [channels, N]; D, dt_bias: [channels]; h0: [batch, channels, N];
    reset: [batch, L] (nonzero = first token of a document).

    Returns (y [batch, channels, L], h_last [batch, channels, N]) in float64,
    plus states [batch, channels, L, N] when return_states is set.
    """
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be [batch, channels, seq]")
    batch, channels, L = x.shape
    A = _f64(A)
    N = A.shape[1]
    dt = _f64(dt, x.shape)
    A = _f64(A, (channels, N))
    B = _f64(B, (batch, N, L))
    C = _f64(C, (batch, N, L))
    D = _f64(D, (channels,))
    z = _f64(z, x.shape)
    dt_bias = _f64(dt_bias, (channels,))
    h0 = _f64(h0, (batch, channels, N))
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)
        if reset.shape != (batch, L):
            raise ValueError("reset must be [batch, seq]")
    y = np.empty((batch, channels, L), dtype=np.float64)
    h_last = np.empty((batch, channels, N), dtype=np.float64)
    states = np.empty((batch, channels, L, N), dtype=np.float64) if return_states else None
    lib = _load()

    def run(rb_re):
        rc = lib.oracle_scan(batch, channels, N, L, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(reset), int(bool(dt_softplus)),
                             _ptr(y), _ptr(h_last), _ptr(states), rb_re[0], rb_re[1])
        if rc != 0:
            raise ValueError("oracle_scan rejected its arguments")

    parts = _split_rows(batch * channels, _threads(threads))
    if len(parts) <= 1:
        for p in parts:
            run(p)
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    if return_states:
        return y, h_last, states
    return y, h_last


def state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, threads=None):
    """Decode step. state: [batch, channels, N] (not modified; the updated
    state is returned); x, dt, z: [batch, channels]; B, C: [batch, N].

    Returns (y [batch, channels], new_state [batch, channels, N]) in float64.
    """
    new_state = np.array(_f64(state), dtype=np.float64, copy=True)
    if new_state.ndim != 3:
        raise ValueError("state must be [batch, channels, state_dim]")
    batch, channels, N = new_state.shape
    x = _f64(x, (batch, channels))
    dt = _f64(dt, (batch, channels))
    A = _f64(A, (channels, N))
    B = _f64(B, (batch, N))
    C = _f64(C, (batch, N))
    D = _f64(D, (channels,))
    z = _f64(z, (batch, channels))
    dt_bias = _f64(dt_bias, (channels,))
    y = np.empty((batch, channels), dtype=np.float64)
    lib = _load()

    def run(rb_re):
        rc = lib.oracle_update(batch, channels, N, _ptr(new_state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(y),
                               rb_re[0], rb_re[1])
        if rc != 0:
            raise ValueError("oracle_update rejected its arguments")

    parts = _split_rows(batch * channels, _threads(threads))
    if len(parts) <= 1:
        for p in parts:
            run(p)
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return y, new_state


def gated_scan(q, k, v, gamma, s0=None, threads=None):
    """Scalar-gated state scan ("Mamba 2 Gated State Scan" problem page):
    S_t = gamma_t S_{t-1} + k_t v_t^T, y_t = q_t^T S_t, from s0 (zeros if None).
    q, k: [batch, L, dk]; v: [batch, L, dv]; gamma: [batch, L];
    s0: [batch, dk, dv]. Returns (y [batch, L, dv], final_state [batch, dk, dv])
    in fp64. Batch items are split over threads; each is one sequential loop."""
    lib = _load()
    q = _f64(q)
    batch, L, dk = q.shape
    dv = np.asarray(v).shape[2]
    k = _f64(k, (batch, L, dk))
    v = _f64(v, (batch, L, dv))
    gamma = _f64(gamma, (batch, L))
    s0 = _f64(s0, (batch, dk, dv))
    y = np.empty((batch, L, dv), dtype=np.float64)
    fs = np.empty((batch, dk, dv), dtype=np.float64)
    if batch == 0:
        return y, fs

    def run(rng):
        rc = lib.oracle_gated_scan(batch, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(s0), _ptr(y),
                                   _ptr(fs), rng[0], rng[1])
        if rc != 0:
            raise ValueError(f"oracle_gated_scan rejected its arguments (code {rc})")

    parts = _split_rows(batch, _threads(threads))
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return y, fs


def effective_attention(dt, A, B, C, dt_bias=None, dt_softplus=True, include_dt_scaling=False,
                        per_state_coord=False, threads=None):
    """Effective attention of the selective scan (TransformerLens "ssm_mixer"
    page, compute_effective_attention):
    M[b, c, i, j] = sum_n C[b, n, i] prod_{k=j+1..i} exp(A[c, n] dt[b, c, k]) B[b, n, j]
    for j <= i, 0 above the diagonal; dt is the step size of the scan
    (softplus(dt + dt_bias) or dt + dt_bias). include_dt_scaling multiplies
    column j by dt[b, c, j] (then y = M x + D x before the gate);
    per_state_coord returns the terms unsummed over n.
    dt: [batch, channels, L]; A: [channels, N]; B, C: [batch, N, L].
    Returns [batch, channels, L, L] or [batch, channels, N, L, L] in fp64."""
    lib = _load()
    dt = _f64(dt)
    batch, channels, L = dt.shape
    A = _f64(A)
    if A.ndim != 2 or A.shape[0] != channels:
        raise ValueError(f"A must be [channels, N], got {A.shape}")
    N = A.shape[1]
    B = _f64(B, (batch, N, L))
    C = _f64(C, (batch, N, L))
    dt_bias = _f64(dt_bias, (channels,))
    shape = (batch, channels, N, L, L) if per_state_coord else (batch, channels, L, L)
    out = np.empty(shape, dtype=np.float64)
    if batch * channels == 0:
        return out

    def run(rng):
        rc = lib.oracle_effective_attention(batch, channels, N, L, _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                            _ptr(dt_bias), int(bool(dt_softplus)), int(bool(include_dt_scaling)),
                                            int(bool(per_state_coord)), _ptr(out), rng[0], rng[1])
        if rc != 0:
            raise ValueError(f"oracle_effective_attention rejected its arguments (code {rc})")

    parts = _split_rows(batch * channels, _threads(threads))
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return out


def _rows_parallel(rows, threads, run):
    parts = _split_rows(rows, _threads(threads))
    if len(parts) == 1:
        run(parts[0])
    elif parts:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))


def conv1d_silu(x_pre, conv_w, conv_b=None, reset=None, threads=None):
    """Causal depthwise conv1d of width W = conv_w.shape[1], then SiLU:
    x[b, c, t] = silu(conv_b[c] + sum_k conv_w[c, k] x_pre[b, c, t - (W-1) + k]),
    taps before position 0 or before the current document's first token
    (reset[b, s] != 0) reading 0. x_pre: [batch, channels, L]; conv_w:
    [channels, W]; conv_b: [channels] or None; reset: [batch, L] or None.
    Returns x [batch, channels, L] in fp64."""
    lib = _load()
    x_pre = _f64(x_pre)
    batch, channels, L = x_pre.shape
    conv_w = _f64(conv_w)
    if conv_w.ndim != 2 or conv_w.shape[0] != channels:
        raise ValueError(f"conv_w must be [channels, W], got {conv_w.shape}")
    W = conv_w.shape[1]
    conv_b = _f64(conv_b, (channels,))
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset, dtype=np.uint8))
        if reset.shape != (batch, L):
            raise ValueError(f"reset must be [batch, L], got {reset.shape}")
    x = np.empty((batch, channels, L), dtype=np.float64)

    def run(rng):
        rc = lib.oracle_conv1d_silu(batch, channels, L, W, _ptr(x_pre), _ptr(conv_w), _ptr(conv_b), _ptr(reset),
                                    _ptr(x), rng[0], rng[1])
        if rc != 0:
            raise ValueError(f"oracle_conv1d_silu rejected its arguments (code {rc})")

    _rows_parallel(batch * channels, threads, run)
    return x


def dt_proj(w_dt, delta, dt_bias=None, apply_softplus=False, threads=None):
    """dt[b, c, t] = sum_k w_dt[c, k] delta[b, t, k]; with apply_softplus,
    softplus(dt + dt_bias[c]). w_dt: [channels, R]; delta: [batch, L, R]
    (token-major). Returns dt [batch, channels, L] in fp64."""
    lib = _load()
    w_dt = _f64(w_dt)
    channels, R = w_dt.shape
    delta = _f64(delta)
    if delta.ndim != 3 or delta.shape[2] != R:
        raise ValueError(f"delta must be [batch, L, {R}], got {delta.shape}")
    batch, L = delta.shape[:2]
    dt_bias = _f64(dt_bias, (channels,))
    dt = np.empty((batch, channels, L), dtype=np.float64)

    def run(rng):
        rc = lib.oracle_dt_proj(batch, channels, L, R, _ptr(w_dt), _ptr(delta), _ptr(dt_bias),
                                int(bool(apply_softplus)), _ptr(dt), rng[0], rng[1])
        if rc != 0:
            raise ValueError(f"oracle_dt_proj rejected its arguments (code {rc})")

    _rows_parallel(batch * channels, threads, run)
    return dt
