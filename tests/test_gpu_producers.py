"""GPU parity of the scan's input-side producers, ss_conv1d_silu and
ss_dt_proj (nnterp "selective_scan" page, class docstring; TransformerLens
"ssm_mixer" page: x is the post-conv SiLU input, dt comes from dt_proj),
against the fp64 oracle on the same seeded inputs, and of the whole chain
conv1d + SiLU -> dt_proj -> scan against the oracle's chain.

Tolerances, from the arithmetic. An output is an fp32 sum of W (conv) or R
(dt_proj) products, then SiLU or softplus (derivatives below 1.1); its
rounding error is at most the number of terms times 2^-24 times the sum of
the terms' magnitudes S, computed here from the inputs. The bar is the
selective scan's pair (fp32 1e-4 / 1e-5, bf16 2e-2 / 1e-4) plus
1.1 (terms + 2) 2^-24 S."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import make_producer_case
from tests.helpers import np64

pytestmark = pytest.mark.gpu

PAIR = {torch.float32: (1e-4, 1e-5), torch.bfloat16: (2e-2, 1e-4)}


def check(got, ref, scale, terms, dtype, what):
    rtol, atol = PAIR[dtype]
    g = np64(got)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = rtol * np.abs(ref) + atol + 1.1 * (terms + 2) * 2.0 ** -24 * scale
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; worst at {i}: "
                             f"gpu {g[i]!r} oracle {ref[i]!r}")


def conv_scale(c):
    """|conv_b| + sum_k |conv_w[c, k]| max_t |x_pre[b, c, t]|, broadcast."""
    xa = np.abs(np64(c["x_pre"])).max(axis=2, keepdims=True)
    return np.abs(np64(c["conv_b"]))[None, :, None] + np.abs(np64(c["conv_w"])).sum(1)[None, :, None] * xa


def dev(c):
    return {k: None if v is None else v.cuda() for k, v in c.items()}


CONV_CASES = [
    # io, batch, channels, L, width, reset mean doc
    ("f32", 2, 3, 37, 4, None),
    ("bf16", 2, 5, 256, 4, None),
    ("bf16", 1, 7, 512, 4, 40),
    ("f32", 2, 3, 64, 8, 10),
    ("bf16", 1, 2, 100, 1, None),
    ("f32", 1, 2, 8, 3, 2),
    ("bf16", 2, 3, 203, 5, 17),
]


@pytest.mark.parametrize("io,batch,channels,L,W,reset", CONV_CASES,
                         ids=[f"{c[0]}-b{c[1]}-c{c[2]}-L{c[3]}-W{c[4]}-r{c[5]}" for c in CONV_CASES])
def test_conv1d_silu_parity(io, batch, channels, L, W, reset):
    print(f"conv1d_silu io={io} b={batch} c={channels} L={L} W={W} reset={reset}", flush=True)
    c = make_producer_case(1400 + L + W, batch, channels, L, W, 16, io, reset_mean_doc=reset)
    d = dev(c)
    x = ss.ss_conv1d_silu(d["x_pre"], d["conv_w"], d["conv_b"], d["reset"])
    torch.cuda.synchronize()
    ref = oracle.conv1d_silu(np64(c["x_pre"]), np64(c["conv_w"]), np64(c["conv_b"]),
                             reset=None if c["reset"] is None else c["reset"].numpy())
    check(x, ref, conv_scale(c), W, x.dtype, "x")


PROJ_CASES = [
    # io, batch, channels, L, rank, apply softplus
    ("f32", 2, 70, 100, 48, False),
    ("bf16", 2, 128, 256, 160, True),
    ("bf16", 1, 64, 64, 40, False),
    ("bf16", 1, 65, 33, 20, True),
    ("f32", 1, 16, 16, 7, False),
    ("f32", 1, 33, 130, 64, True),
    ("bf16", 1, 100, 200, 64, True),     # tiled form: channel and token tails
    ("f32", 2, 64, 96, 128, False),      # tiled form: 8 chunks of k
    ("bf16", 1, 70, 72, 256, True),
]


@pytest.mark.parametrize("io,batch,channels,L,R,apply", PROJ_CASES,
                         ids=[f"{c[0]}-b{c[1]}-c{c[2]}-L{c[3]}-R{c[4]}-sp{int(c[5])}" for c in PROJ_CASES])
def test_dt_proj_parity(io, batch, channels, L, R, apply):
    print(f"dt_proj io={io} b={batch} c={channels} L={L} R={R} apply={apply}", flush=True)
    c = make_producer_case(1500 + L + R, batch, channels, L, 4, R, io)
    d = dev(c)
    dt = ss.ss_dt_proj(d["w_dt"], d["delta"], d["dt_bias"], apply_softplus=apply)
    torch.cuda.synchronize()
    w, delta = np64(c["w_dt"]), np64(c["delta"])
    ref = oracle.dt_proj(w, delta, dt_bias=np64(c["dt_bias"]), apply_softplus=apply)
    scale = np.stack([np.abs(w) @ np.abs(delta[b]).T for b in range(batch)])
    check(dt, ref, scale, R, dt.dtype, "dt")


@pytest.mark.parametrize("io,R", [("bf16", 160), ("f32", 64)])
def test_dt_proj_long_runs(io, R, monkeypatch):
    """The tiled form with its grid capped at 7 blocks (SS_DT_PROJ_BLOCKS), so
    that every block walks a long run of (batch row, 256-channel group,
    64-token) units, crossing batch rows, channel groups (the last one
    partial: 600 = 2 x 256 + 88) and the partial last token unit (1000 = 15 x
    64 + 40); every output against the oracle."""
    print(f"dt_proj long runs io={io} R={R}", flush=True)
    monkeypatch.setenv("SS_DT_PROJ_BLOCKS", "7")
    c = make_producer_case(1560 + R, 2, 600, 1000, 4, R, io)
    d = dev(c)
    dt = ss.ss_dt_proj(d["w_dt"], d["delta"], d["dt_bias"], apply_softplus=True)
    torch.cuda.synchronize()
    w, delta = np64(c["w_dt"]), np64(c["delta"])
    ref = oracle.dt_proj(w, delta, dt_bias=np64(c["dt_bias"]), apply_softplus=True)
    scale = np.stack([np.abs(w) @ np.abs(delta[b]).T for b in range(2)])
    check(dt, ref, scale, R, dt.dtype, "dt")


def test_dt_proj_full_size_sampled():
    """A Mamba-2.8B-shaped projection for one batch row: channels 5120, rank
    160, seq 2048, bf16, with bias and softplus; sampled channels."""
    print("dt_proj full size 1x5120x2048 R160", flush=True)
    c = make_producer_case(1590, 1, 5120, 2048, 4, 160, "bf16")
    d = dev(c)
    dt = ss.ss_dt_proj(d["w_dt"], d["delta"], d["dt_bias"], apply_softplus=True)
    dt2 = ss.ss_dt_proj(d["w_dt"], d["delta"], d["dt_bias"], apply_softplus=True)
    torch.cuda.synchronize()
    assert torch.equal(dt, dt2), "not bitwise reproducible"
    rows = [0, 1, 63, 64, 2500, 5119]
    w, delta = np64(c["w_dt"])[rows], np64(c["delta"])
    ref = oracle.dt_proj(w, delta, dt_bias=np64(c["dt_bias"])[rows], apply_softplus=True)
    scale = (np.abs(w) @ np.abs(delta[0]).T)[None]
    check(dt[:, rows], ref, scale, 160, torch.bfloat16, "dt sampled channels")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chain_into_the_scan(io):
    """conv1d + SiLU -> dt_proj (raw) -> ss_scan_fwd with softplus(dt + bias),
    against the oracle's chain on the same inputs. The scan consumes the
    GPU's x and dt, so the oracle's scan is run on those too (the producers
    are checked above); the last line checks the chain's x and dt."""
    print(f"producer chain io={io}", flush=True)
    from selective_state_space_ss_amd.workloads import make_case
    batch, channels, N, L, R = 2, 24, 16, 300, 32
    c = make_producer_case(1600, batch, channels, L, 4, R, io, reset_mean_doc=90)
    s = make_case(1601, batch, channels, N, L, io, gate=True, h0=False)
    d, sd = dev(c), dev(s)
    x = ss.ss_conv1d_silu(d["x_pre"], d["conv_w"], d["conv_b"], d["reset"])
    dt = ss.ss_dt_proj(d["w_dt"], d["delta"])
    y, h = ss.ss_scan_fwd(x, dt, sd["A"], sd["B"], sd["C"], D=sd["D"], z=sd["z"], dt_bias=d["dt_bias"],
                          reset=d["reset"])
    torch.cuda.synchronize()
    yr, hr = oracle.scan(np64(x), np64(dt), np64(s["A"]), np64(s["B"]), np64(s["C"]), D=np64(s["D"]),
                         z=np64(s["z"]), dt_bias=np64(c["dt_bias"]), reset=c["reset"].numpy())
    rtol, atol = PAIR[x.dtype]
    assert np.allclose(np64(y), yr, rtol=rtol, atol=atol), float(np.abs(np64(y) - yr).max())
    assert np.allclose(np64(h), hr, rtol=1e-4, atol=1e-5), float(np.abs(np64(h) - hr).max())
    xr = oracle.conv1d_silu(np64(c["x_pre"]), np64(c["conv_w"]), np64(c["conv_b"]), reset=c["reset"].numpy())
    dtr = oracle.dt_proj(np64(c["w_dt"]), np64(c["delta"]))
    assert np.allclose(np64(x), xr, rtol=rtol, atol=atol) and np.allclose(np64(dt), dtr, rtol=rtol, atol=atol)


def test_producer_edges():
    """Zero-size calls are no-ops; a rank beyond the tiled form (300 > 8
    chunks of 32) and a row length that is not a whole vector take the
    general path; width 8 with a reset on every token reads only the token
    itself."""
    print("producer edges", flush=True)
    c = dev(make_producer_case(1700, 1, 4, 0, 4, 16, "bf16"))
    assert ss.ss_conv1d_silu(c["x_pre"], c["conv_w"], c["conv_b"]).shape == (1, 4, 0)
    assert ss.ss_dt_proj(c["w_dt"], c["delta"]).shape == (1, 4, 0)
    for L, R in ((64, 300), (37, 64)):
        c = make_producer_case(1701 + L, 2, 40, L, 4, R, "bf16")
        d = dev(c)
        dt = ss.ss_dt_proj(d["w_dt"], d["delta"], d["dt_bias"], apply_softplus=True)
        torch.cuda.synchronize()
        w, delta = np64(c["w_dt"]), np64(c["delta"])
        ref = oracle.dt_proj(w, delta, dt_bias=np64(c["dt_bias"]), apply_softplus=True)
        scale = np.stack([np.abs(w) @ np.abs(delta[b]).T for b in range(2)])
        check(dt, ref, scale, R, torch.bfloat16, f"dt L={L} R={R}")
    c = make_producer_case(1703, 1, 3, 40, 8, 16, "f32")
    c["reset"] = torch.ones(1, 40, dtype=torch.uint8)
    d = dev(c)
    x = ss.ss_conv1d_silu(d["x_pre"], d["conv_w"], d["conv_b"], d["reset"])
    torch.cuda.synchronize()
    pre = np64(c["conv_w"])[:, -1][None, :, None] * np64(c["x_pre"]) + np64(c["conv_b"])[None, :, None]
    check(x, pre / (1.0 + np.exp(-pre)), np.abs(pre) + 1.0, 1, torch.float32, "x, reset on every token")
