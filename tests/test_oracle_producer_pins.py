"""Pins of the oracle's input-side producers of the scan (nnterp
"selective_scan" page, class docstring: x is the causal conv1d output after
SiLU and dt the dt_proj output; TransformerLens "ssm_mixer" page: x is the
post-conv SiLU input, dt read from dt_proj's output) against routes of their
own: numpy.convolve, the impulse response, per-document concatenation, the
width-1 case, numpy matmul, the identity projection."""
import numpy as np
import pytest

import oracle


def silu(v):
    return v / (1.0 + np.exp(-v))


def conv_case(seed, batch=2, channels=3, L=19, W=4):
    rng = np.random.default_rng(seed)
    return dict(x_pre=rng.standard_normal((batch, channels, L)), w=rng.standard_normal((channels, W)),
                b=rng.standard_normal(channels))


def close(a, b, rtol=1e-13, atol=1e-13):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


@pytest.mark.parametrize("W", [1, 2, 4, 7])
def test_ppin1_matches_numpy_convolve(W):
    """Without resets the pre-activation is numpy.convolve(x_pre, w reversed)
    cut to the first L outputs (full convolution = zero left padding)."""
    c = conv_case(21 + W, W=W)
    x = oracle.conv1d_silu(c["x_pre"], c["w"], c["b"])
    batch, channels, L = c["x_pre"].shape
    for b in range(batch):
        for ch in range(channels):
            pre = np.convolve(c["x_pre"][b, ch], c["w"][ch][::-1])[:L] + c["b"][ch]
            close(x[b, ch], silu(pre))


def test_ppin2_impulse_response():
    """x_pre = 1 at one position t0: the pre-activation at t0 + m is
    b + w[W-1-m] for 0 <= m < W (the newest tap, w[W-1], meets the current
    token) and b elsewhere."""
    W, L, t0 = 4, 12, 5
    c = conv_case(22, batch=1, channels=2, L=L, W=W)
    x_pre = np.zeros((1, 2, L))
    x_pre[0, :, t0] = 1.0
    x = oracle.conv1d_silu(x_pre, c["w"], c["b"])
    for ch in range(2):
        pre = np.full(L, c["b"][ch])
        for m in range(W):
            pre[t0 + m] += c["w"][ch, W - 1 - m]
        close(x[0, ch], silu(pre))


def test_ppin3_reset_restarts_the_convolution():
    """With document starts marked, each document is convolved as if it were
    its own sequence: the packed result is the concatenation of per-document
    results without resets."""
    c = conv_case(23, batch=2, channels=2, L=20, W=4)
    reset = np.zeros((2, 20), dtype=np.uint8)
    starts = {0: [0, 3, 11, 12], 1: [0, 17]}
    for b, ss in starts.items():
        reset[b, ss] = 1
    x = oracle.conv1d_silu(c["x_pre"], c["w"], c["b"], reset=reset)
    for b, ss in starts.items():
        bounds = ss + [20]
        for s0, s1 in zip(bounds[:-1], bounds[1:]):
            part = oracle.conv1d_silu(c["x_pre"][b:b + 1, :, s0:s1], c["w"], c["b"])
            close(x[b:b + 1, :, s0:s1], part, rtol=0, atol=0)
    # a reset at t = 0 changes nothing
    close(oracle.conv1d_silu(c["x_pre"], c["w"], c["b"], reset=np.eye(1, 20, 0, dtype=np.uint8).repeat(2, 0)),
          oracle.conv1d_silu(c["x_pre"], c["w"], c["b"]), rtol=0, atol=0)


def test_ppin4_width_one_is_elementwise():
    c = conv_case(24, W=1)
    x = oracle.conv1d_silu(c["x_pre"], c["w"], None)
    close(x, silu(c["w"][None, :, 0:1] * c["x_pre"]))


@pytest.mark.parametrize("apply", [False, True])
def test_ppin5_dt_proj_matches_numpy_matmul(apply):
    """dt[b] = w_dt @ delta[b]^T; applied: softplus(dt + bias) via
    numpy.logaddexp."""
    rng = np.random.default_rng(25)
    w = rng.standard_normal((6, 5))
    delta = rng.standard_normal((2, 9, 5))
    bias = rng.standard_normal(6)
    dt = oracle.dt_proj(w, delta, dt_bias=bias, apply_softplus=apply)
    ref = np.stack([w @ delta[b].T for b in range(2)])
    if apply:
        ref = np.logaddexp(0.0, ref + bias[None, :, None])
    close(dt, ref, rtol=1e-12, atol=1e-12)


def test_ppin6_identity_projection_is_a_transpose():
    """w_dt = I (channels = rank): dt[b, c, t] = delta[b, t, c] exactly."""
    rng = np.random.default_rng(26)
    delta = rng.standard_normal((2, 7, 4))
    dt = oracle.dt_proj(np.eye(4), delta)
    close(dt, delta.transpose(0, 2, 1), rtol=0, atol=0)


def test_ppin7_chain_feeds_the_scan():
    """The producers compose with the scan: x = conv1d_silu(x_pre) and raw dt
    = dt_proj(delta) with the scan's softplus(dt + bias) give the same y as
    dt already activated by dt_proj (apply_softplus) with the scan's softplus
    off."""
    rng = np.random.default_rng(27)
    batch, channels, N, L, R = 2, 3, 4, 15, 5
    x = oracle.conv1d_silu(rng.standard_normal((batch, channels, L)), rng.standard_normal((channels, 4)),
                           rng.standard_normal(channels))
    w = rng.standard_normal((channels, R)) * 0.3
    delta = rng.standard_normal((batch, L, R))
    bias = rng.uniform(-3, -1, channels)
    A = -rng.uniform(0.5, 2.0, (channels, N))
    Bm, Cm = rng.standard_normal((batch, N, L)), rng.standard_normal((batch, N, L))
    y1, h1 = oracle.scan(x, oracle.dt_proj(w, delta), A, Bm, Cm, dt_bias=bias, dt_softplus=True)
    y2, h2 = oracle.scan(x, oracle.dt_proj(w, delta, dt_bias=bias, apply_softplus=True), A, Bm, Cm,
                         dt_softplus=False)
    close(y1, y2, rtol=1e-12, atol=1e-12)
    close(h1, h2, rtol=1e-12, atol=1e-12)
