"""GPU parity of ss_scan_fwd_conv, the scan with the causal conv1d + SiLU
fused in (nnterp "selective_scan" page, class docstring: the scan's x is the
conv1d output after SiLU; TransformerLens "ssm_mixer" page: x is the post-conv
SiLU input), against the oracle's chain oracle.conv1d_silu -> oracle.scan on
the same seeded inputs, element by element.

The fused kernel keeps x in fp32 (never rounded to the I/O type), so the
oracle's chain, fp64 throughout, is the reference; the bar is the scan's
(fp32 I/O 1e-4 / 1e-5, bf16 2e-2 / 1e-4; final state at the fp32 bar). The
conv's own fp32 rounding (at most (W + 2) 2^-24 times the sum of its terms'
magnitudes, about 1e-7 here) enters y through dt * x * B with dt ~ 0.02, far
below those bars."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import make_case, make_inputs, make_producer_case
from tests.helpers import TOL, TOL_STATE, check_close, np64, to_dev

pytestmark = pytest.mark.gpu


def conv_inputs(seed, batch, channels, L, width, io, reset=None):
    """x_pre, conv_w, conv_b with the producer recipe."""
    pc = make_producer_case(seed, batch, channels, L, width, 1, io)
    return pc["x_pre"], pc["conv_w"], pc["conv_b"]


def oracle_chain(inp, x_pre, conv_w, conv_b, dt_softplus=True):
    reset = None if inp.get("reset") is None else inp["reset"].numpy()
    x = oracle.conv1d_silu(np64(x_pre), np64(conv_w), np64(conv_b), reset=reset)
    return oracle.scan(x, np64(inp["dt"]), np64(inp["A"]), np64(inp["B"]), np64(inp["C"]), D=np64(inp["D"]),
                       z=np64(inp.get("z")), dt_bias=np64(inp["dt_bias"]), h0=np64(inp.get("h0")), reset=reset,
                       dt_softplus=dt_softplus)


def run_fused(inp, x_pre, conv_w, conv_b, dt_softplus=True):
    d = to_dev(inp)
    y, h = ss.ss_scan_fwd_conv(x_pre.cuda(), d["dt"], d["A"], d["B"], d["C"], conv_w.cuda(),
                               None if conv_b is None else conv_b.cuda(), D=d["D"], z=d.get("z"),
                               dt_bias=d["dt_bias"], h0=d.get("h0"), reset=d.get("reset"), dt_softplus=dt_softplus)
    torch.cuda.synchronize()
    return y, h


CASES = [
    # io, L, width, gate, h0, reset (mean doc length, "every", "edges" or None), N
    ("bf16", 2048, 4, True, True, None, 16), ("bf16", 2048, 4, True, False, 200, 16),
    ("f32", 1000, 4, True, True, None, 16), ("f32", 257, 3, False, True, 30, 16),
    ("bf16", 1, 4, True, True, None, 16), ("bf16", 7, 2, True, False, 3, 16), ("f32", 15, 1, True, True, None, 4),
    ("bf16", 255, 5, False, False, None, 16), ("bf16", 513, 8, True, True, 40, 16), ("f32", 256, 8, True, False, 16, 4),
    ("bf16", 1100, 4, True, True, "every", 16), ("f32", 1100, 4, True, True, "edges", 16),
    ("bf16", 1100, 7, False, True, "edges", 16), ("bf16", 600, 4, True, True, 50, 33),
    ("f32", 300, 6, True, True, None, 64), ("bf16", 4100, 4, True, True, 512, 16),
]


def _mask(kind, batch, L):
    m = torch.zeros(batch, L, dtype=torch.uint8)
    t = torch.arange(L)
    if kind == "every":
        m[:] = 1
    else:  # lane (16-token) and chunk (256-token) edges, and pairs across them
        m[:, t % 16 == 0] = 1
        for e in (256, 512, 768, 1024):
            if e < L:
                m[:, e - 1:e + 1] = 1
    return m


@pytest.mark.parametrize("io,L,width,gate,h0,reset,N", CASES,
                         ids=[f"{c[0]}-L{c[1]}-W{c[2]}-g{int(c[3])}-h{int(c[4])}-r{c[5]}-N{c[6]}" for c in CASES])
def test_fused_conv_parity(io, L, width, gate, h0, reset, N):
    print(f"fused conv io={io} L={L} W={width} gate={gate} h0={h0} reset={reset} N={N}", flush=True)
    mean = reset if isinstance(reset, int) else None
    inp = make_case(700 + L + width, 2, 19, N, L, io, gate=gate, h0=h0, reset_mean_doc=mean)
    if isinstance(reset, str):
        inp["reset"] = _mask(reset, 2, L)
    x_pre, conv_w, conv_b = conv_inputs(800 + L + width, 2, 19, L, width, io)
    y, h = run_fused(inp, x_pre, conv_w, conv_b)
    yr, hr = oracle_chain(inp, x_pre, conv_w, conv_b)
    check_close(np64(y), yr, *TOL[io], f"y fused {io} L={L} W={width}")
    check_close(np64(h), hr, *TOL_STATE, f"h_last fused {io} L={L} W={width}")


def test_fused_conv_without_bias_and_softplus_off():
    inp = make_case(790, 1, 21, 16, 700, "f32", gate=False, h0=False)
    inp["dt"] = (inp["dt"].abs() * 0.05).contiguous()
    inp["dt_bias"] = None
    x_pre, conv_w, _ = conv_inputs(791, 1, 21, 700, 4, "f32")
    y, h = run_fused(inp, x_pre, conv_w, None, dt_softplus=False)
    yr, hr = oracle_chain(inp, x_pre, conv_w, None, dt_softplus=False)
    check_close(np64(y), yr, *TOL["f32"], "y fused, no bias, softplus off")
    check_close(np64(h), hr, *TOL_STATE, "h_last fused, no bias, softplus off")


@pytest.mark.parametrize("reset", [False, True])
def test_fused_conv_full_size_every_element(reset):
    """The Mamba-2.8B layer shape (batch 8, channels 5120, seq 2048, bf16,
    gate, h0; width 4), with and without a packed-sequence reset mask; every
    element of y and h_last against the oracle's chain over every row."""
    print(f"fused conv full size reset={reset}", flush=True)
    inp = make_inputs("mamba2p8b")
    if reset:
        inp["reset"] = make_case(795, 8, 1, 16, 2048, reset_mean_doc=512)["reset"]
    x_pre, conv_w, conv_b = conv_inputs(796, 8, 5120, 2048, 4, "bf16")
    y, h = run_fused(inp, x_pre, conv_w, conv_b)
    yr, hr = oracle_chain(inp, x_pre, conv_w, conv_b)
    check_close(np64(y), yr, *TOL["bf16"], f"y fused full size reset={reset}")
    check_close(np64(h), hr, *TOL_STATE, f"h_last fused full size reset={reset}")


def test_fused_matches_two_kernel_chain():
    """The fused call against ss_conv1d_silu -> ss_scan_fwd on the GPU. The
    two-kernel chain rounds x to bf16 between its kernels (2^-9 relative), so
    elementwise the two differ near y = 0; normwise they agree to about that
    rounding, and the fused call holds the elementwise bar against the
    oracle's chain."""
    inp = make_case(797, 2, 64, 16, 1500, "bf16", gate=True, h0=True, reset_mean_doc=300)
    x_pre, conv_w, conv_b = conv_inputs(798, 2, 64, 1500, 4, "bf16")
    yf, hf = run_fused(inp, x_pre, conv_w, conv_b)
    d = to_dev(inp)
    x = ss.ss_conv1d_silu(x_pre.cuda(), conv_w.cuda(), conv_b.cuda(), d["reset"])
    y2, h2 = ss.ss_scan_fwd(x, d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], dt_bias=d["dt_bias"],
                            h0=d["h0"], reset=d["reset"])
    torch.cuda.synchronize()
    yr, hr = oracle_chain(inp, x_pre, conv_w, conv_b)
    check_close(np64(yf), yr, *TOL["bf16"], "fused vs oracle chain, y")
    check_close(np64(hf), hr, *TOL_STATE, "fused vs oracle chain, h_last")
    norm = lambda a: float(np.linalg.norm(a.ravel()))
    for got, ref, what in ((np64(y2), yr, "two kernels vs oracle, y"), (np64(yf), np64(y2), "fused vs two kernels, y"),
                           (np64(h2), hr, "two kernels vs oracle, h_last"),
                           (np64(hf), np64(h2), "fused vs two kernels, h_last")):
        rel = norm(got - ref) / norm(ref)
        assert rel < 4e-3, f"{what}: normwise relative difference {rel:.3g}"
    # the fused call is the closer of the two to the oracle
    assert norm(np64(yf) - yr) <= norm(np64(y2) - yr)


def test_fused_conv_errors():
    inp = to_dev(make_case(799, 1, 8, 16, 64, "bf16"))
    x_pre, conv_w, _ = conv_inputs(799, 1, 8, 64, 4, "bf16")
    wide = torch.zeros(8, 9, device="cuda")
    with pytest.raises(ss.SSError) as e:
        ss.ss_scan_fwd_conv(x_pre.cuda(), inp["dt"], inp["A"], inp["B"], inp["C"], wide)
    assert e.value.code == 4
    with pytest.raises(ValueError):
        ss.ss_scan_fwd_conv(x_pre.cuda(), inp["dt"], inp["A"], inp["B"], inp["C"], conv_w.cuda()[:4])
