"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on
the five workloads and on ragged and degenerate shapes.

Tolerances (tests/helpers.py): fp32 I/O |d| <= 1e-5 + 1e-4 |ref|; bf16 I/O
|d| <= 1e-4 + 2e-2 |ref|; the fp32 final / cached state at the fp32 bar.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import WORKLOADS, make_case, make_decode_case, make_inputs
from tests.helpers import (RESET_SCAN_KERNELS, SCAN_KERNELS, TOL, TOL_STATE, check_close, force_scan_kernel,
                           io_name, np64, oracle_scan_full, oracle_scan_rows, sample_rows, to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(params=SCAN_KERNELS)
def scan_kernel(request, monkeypatch):
    """Every prompt-scan kernel variant (tests/helpers.py, SCAN_KERNELS)."""
    force_scan_kernel(monkeypatch, request.param)
    return request.param


@pytest.fixture(params=RESET_SCAN_KERNELS)
def reset_scan_kernel(request, monkeypatch):
    """The variants that take a reset mask."""
    force_scan_kernel(monkeypatch, request.param)
    return request.param


def run_scan(inp, dt_softplus=True, **kw):
    d = to_dev(inp)
    y, h = ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d.get("z"), dt_bias=d["dt_bias"],
                          h0=d.get("h0"), reset=d.get("reset"), dt_softplus=dt_softplus, **kw)
    torch.cuda.synchronize()
    return y, h


def compare_full(inp, dt_softplus=True, what=""):
    y, h = run_scan(inp, dt_softplus)
    yr, hr = oracle_scan_full(inp, dt_softplus)
    rtol, atol = TOL[io_name(inp["x"])]
    s = check_close(np64(y), yr, rtol, atol, f"y {what}")
    check_close(np64(h), hr, *TOL_STATE, f"h_last {what}")
    return s


# ------------------------------------------------------------------ workloads
def test_workload_tiny_fp32():
    inp = make_inputs("tiny_fp32")
    print("workload tiny_fp32", flush=True)
    compare_full(inp, what="tiny_fp32")


# The oracle's results for the full-size workloads, computed once per module
# and shared by every kernel variant that is compared with them.
_FULL = {}


def full_size_reference(name):
    if name not in _FULL:
        inp = make_inputs(name)
        print(f"oracle over every row of {name}", flush=True)
        yr, hr = oracle_scan_full(inp)
        _FULL[name] = (inp, yr, hr)
    return _FULL[name]


@pytest.mark.parametrize("name", ["mamba130m", "mamba2p8b", "packed_reset"])
def test_workload_full_size_every_element(name, scan_kernel):
    """The full-size launch (the benchmark's), every element of y and h_last
    against the oracle run over every row."""
    w = WORKLOADS[name]
    print(f"workload {name} full size, {scan_kernel} kernel", flush=True)
    inp, yr, hr = full_size_reference(name)
    y, h = run_scan(inp)
    rtol, atol = TOL[w.io_dtype]
    check_close(np64(y), yr, rtol, atol, f"y {name}")
    check_close(np64(h), hr, *TOL_STATE, f"h_last {name}")


def test_packed_reset_default_kernel_choice(monkeypatch):
    """The library's own choice of tokens per lane (no override): with a reset
    mask and a long sequence on few channels it takes 32 tokens per lane;
    every element against the oracle. (Its choice of the few-row forms is
    test_mamba130m_default_kernel_choice.)"""
    for k in ("SS_SCAN_TOKENS_PER_LANE", "SS_SCAN_KERNEL", "SS_SCAN_FORM"):
        monkeypatch.delenv(k, raising=False)
    print("default kernel choice: bf16 1 x 64 x 16 x 8192 with resets", flush=True)
    inp = make_case(905, 1, 64, 16, 8192, "bf16", gate=True, h0=True, reset_mean_doc=512)
    compare_full(inp, what="default choice 1x64x8192")
    inp, yr, hr = full_size_reference("packed_reset")
    y, h = run_scan(inp)
    check_close(np64(y), yr, *TOL["bf16"], "y packed_reset default choice")
    check_close(np64(h), hr, *TOL_STATE, "h_last packed_reset default choice")


def test_mamba130m_default_kernel_choice(monkeypatch):
    """The library's own choice of form (no override) at the Mamba-130M layer
    shape, where it gives each channel row 32 lanes, and at 1 x 3072
    channels, where it gives 64; every element against the oracle."""
    for k in ("SS_SCAN_TOKENS_PER_LANE", "SS_SCAN_KERNEL", "SS_SCAN_FORM"):
        monkeypatch.delenv(k, raising=False)
    print("default kernel choice: mamba130m full size", flush=True)
    inp, yr, hr = full_size_reference("mamba130m")
    y, h = run_scan(inp)
    check_close(np64(y), yr, *TOL["bf16"], "y mamba130m default choice")
    check_close(np64(h), hr, *TOL_STATE, "h_last mamba130m default choice")
    print("default kernel choice: bf16 1 x 3072 x 16 x 2048", flush=True)
    inp = make_case(906, 1, 3072, 16, 2048, "bf16", gate=True, h0=True)
    compare_full(inp, what="default choice 1x3072x2048")


def _edge_mask(kind, batch, L):
    """Deterministic reset masks on the kernels' lane and chunk edges (16 or
    32 tokens per lane, 16 lanes per chunk)."""
    m = torch.zeros(batch, L, dtype=torch.uint8)
    t = torch.arange(L)
    if kind == "every_token":
        m[:] = 1
    elif kind == "lane16":
        m[:, t % 16 == 0] = 1
    elif kind == "chunk256":
        m[:, t % 256 == 0] = 1
    elif kind == "lane32":
        m[:, t % 32 == 0] = 1
    elif kind == "chunk512":
        m[:, t % 512 == 0] = 1
    elif kind == "straddle":
        for e in (256, 512, 768, 1024):      # two adjacent resets across each chunk edge
            if e < L:
                m[:, e - 1:e + 1] = 1
        m[:, 15:17] = 1                       # and across a lane edge
    elif kind == "first_only":
        m[:, 0] = 1
    elif kind == "last_only":
        m[:, L - 1] = 1
    elif kind == "lane_ends":
        m[:, (t % 16 == 15) | (t % 32 == 31)] = 1
    else:
        raise ValueError(kind)
    return m


EDGE_KINDS = ["every_token", "lane16", "chunk256", "lane32", "chunk512", "straddle", "first_only", "last_only",
              "lane_ends"]


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("kind", EDGE_KINDS)
def test_reset_edges(kind, io, reset_scan_kernel):
    """Resets placed on every token, on lane and chunk boundaries, in adjacent
    pairs straddling them, and with an initial state ("s6_reset" post,
    Enforced Boundary Resetting: the state is zeroed before a document's
    first token; a reset at t = 0 discards h0)."""
    print(f"reset edges {kind} io={io} kernel={reset_scan_kernel}", flush=True)
    L = 1100
    inp = make_case(920 + EDGE_KINDS.index(kind), 2, 19, 16, L, io, gate=True, h0=True)
    inp["reset"] = _edge_mask(kind, 2, L)
    compare_full(inp, what=f"reset {kind} {io}")


@pytest.mark.parametrize("N", [32, 64])
def test_wide_state_long_sequence(N):
    """state_dim 32 and 64 over several chunks with a ragged tail: the
    coordinate groups staged one after another, the carry of each."""
    print(f"wide state N={N}", flush=True)
    inp = make_case(320 + N, 2, 40, N, 1100, "bf16", gate=True, h0=True, reset_mean_doc=200)
    compare_full(inp, what=f"N={N} L=1100")


def test_workload_decode_full():
    w = WORKLOADS["decode"]
    print("workload decode", flush=True)
    inp = make_inputs("decode")
    d = to_dev(inp)
    state = d["state"].clone()
    y = ss.ss_state_update(state, d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                           dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    yr, sr = oracle.state_update(np64(inp["state"]), np64(inp["x"]), np64(inp["dt"]), np64(inp["A"]),
                                 np64(inp["B"]), np64(inp["C"]), D=np64(inp["D"]), z=np64(inp["z"]),
                                 dt_bias=np64(inp["dt_bias"]))
    check_close(np64(y), yr, *TOL[w.io_dtype], "decode y")
    check_close(np64(state), sr, *TOL_STATE, "decode state")


# ------------------------------------------------------------------ ragged / tiles
RAGGED = [
    # io, L, gate, h0, reset
    ("f32", 1, False, False, None), ("f32", 7, True, True, None), ("f32", 255, True, False, None),
    ("f32", 256, False, True, 16), ("f32", 257, True, True, 8), ("f32", 1000, True, True, None),
    ("bf16", 1, True, True, None), ("bf16", 15, False, False, 4), ("bf16", 511, True, True, None),
    ("bf16", 512, True, True, None), ("bf16", 513, True, False, None), ("bf16", 1024, False, True, 64),
    ("bf16", 1543, True, True, None), ("bf16", 2048, True, True, None), ("bf16", 2049, False, False, 100),
    ("bf16", 4100, True, True, 512),
    # even lengths whose last 16-token tile is partial (the row-parallel walk's tail)
    ("f32", 2, True, True, None), ("bf16", 14, True, False, 4), ("f32", 18, False, True, 6),
    ("bf16", 258, True, True, 50), ("bf16", 1030, False, True, None),
]


@pytest.mark.parametrize("io,L,gate,h0,reset", RAGGED, ids=[f"{r[0]}-L{r[1]}-g{int(r[2])}-h{int(r[3])}-r{r[4]}"
                                                            for r in RAGGED])
def test_ragged_shapes(io, L, gate, h0, reset, scan_kernel):
    """Chunks of 256 or 512 tokens, a ragged tail, channels not a multiple of
    the block's 16."""
    print(f"ragged io={io} L={L} gate={gate} h0={h0} reset={reset}", flush=True)
    inp = make_case(100 + L, 2, 19, 16, L, io, gate=gate, h0=h0, reset_mean_doc=reset)
    compare_full(inp, what=f"{io} L={L}")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17, 24, 31, 32, 33, 48, 63, 64])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_state_dims(io, N, scan_kernel):
    print(f"state_dim io={io} N={N}", flush=True)
    inp = make_case(200 + N, 3, 5, N, 300, io, gate=True, h0=True, reset_mean_doc=50)
    compare_full(inp, what=f"{io} N={N}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_channel_blocks_and_ragged_tail(io, scan_kernel):
    """Several 64-row blocks with a partial last one, and a partial tile."""
    print(f"channels=200 io={io}", flush=True)
    inp = make_case(310, 2, 200, 16, 334, io, gate=True, h0=True, reset_mean_doc=40)
    compare_full(inp, what=f"{io} channels=200")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_unaligned_inputs(io, scan_kernel):
    """Tensors that start one element past an aligned address: the library
    takes its unvectorised paths and the results do not change."""
    print(f"unaligned io={io}", flush=True)
    inp = make_case(311, 2, 70, 16, 130, io, gate=True, h0=True, reset_mean_doc=30)
    compare_full(inp, what=f"{io} aligned")
    d = to_dev(inp)
    shifted = {}
    for k in ("x", "dt", "z", "B", "C"):
        t = d[k]
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        shifted[k] = v
    y, h = ss.ss_scan_fwd(shifted["x"], shifted["dt"], d["A"], shifted["B"], shifted["C"], D=d["D"], z=shifted["z"],
                          dt_bias=d["dt_bias"], h0=d["h0"], reset=d["reset"])
    torch.cuda.synchronize()
    yr, hr = oracle_scan_full(inp, True)
    check_close(np64(y), yr, *TOL[io], f"y unaligned {io}")
    check_close(np64(h), hr, *TOL_STATE, f"h_last unaligned {io}")


def test_softplus_off_and_optional_inputs_absent(scan_kernel):
    inp = make_case(301, 2, 17, 16, 600, "f32", gate=False, h0=False)
    inp["D"] = None
    inp["dt_bias"] = None
    inp["dt"] = (inp["dt"].abs() * 0.05).contiguous()  # a positive step size without softplus
    y, h = run_scan(inp, dt_softplus=False)
    yr, hr = oracle.scan(np64(inp["x"]), np64(inp["dt"]), np64(inp["A"]), np64(inp["B"]), np64(inp["C"]),
                         dt_softplus=False)
    check_close(np64(y), yr, *TOL["f32"], "y softplus off")
    check_close(np64(h), hr, *TOL_STATE, "h_last softplus off")


def test_seqlen_zero_returns_initial_state(scan_kernel):
    inp = make_case(302, 2, 5, 16, 0, "bf16", gate=True, h0=True)
    y, h = run_scan(inp)
    assert y.numel() == 0
    assert torch.equal(h.cpu(), inp["h0"])
    inp["h0"] = None
    _, h = run_scan(inp)
    assert torch.count_nonzero(h) == 0


def test_empty_batch_and_channels_are_noops():
    for b, c in [(0, 5), (2, 0)]:
        inp = make_case(303, b, c, 16, 32, "bf16")
        y, h = run_scan(inp)
        assert y.numel() == 0 and h.numel() == 0


# ------------------------------------------------------------------ numerics
def test_softplus_accuracy(scan_kernel):
    """L = 1, N = 1, B = C = x = 1, zero state: y = dt = softplus(dt_raw)."""
    v = torch.linspace(-30, 30, 6001, dtype=torch.float32)
    ch = v.numel()
    inp = dict(x=torch.ones(1, ch, 1), dt=v.view(1, ch, 1).clone(), A=-torch.ones(ch, 1), B=torch.ones(1, 1, 1),
               C=torch.ones(1, 1, 1), D=None, z=None, dt_bias=None, h0=None, reset=None)
    y, _ = run_scan(inp)
    ref = np.logaddexp(0.0, v.double().numpy())
    check_close(np64(y)[0, :, 0], ref, 2e-6, 1e-30, "softplus")


def test_gate_accuracy(scan_kernel):
    """B = 0, D = 1, x = 1: y = silu(z)."""
    z = torch.linspace(-40, 40, 8001, dtype=torch.float32)
    ch = z.numel()
    inp = dict(x=torch.ones(1, ch, 1), dt=torch.zeros(1, ch, 1), A=-torch.ones(ch, 1), B=torch.zeros(1, 1, 1),
               C=torch.ones(1, 1, 1), D=torch.ones(ch), z=z.view(1, ch, 1).clone(), dt_bias=None, h0=None,
               reset=None)
    y, _ = run_scan(inp)
    zz = z.double().numpy()
    ref = zz / (1.0 + np.exp(-zz))
    check_close(np64(y)[0, :, 0], ref, 2e-6, 1e-30, "silu")


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,gate", [(1, True), (3, False), (4, True), (9, True), (16, False), (16, True), (17, True),
                                    (32, True), (33, False), (48, True), (64, True), (64, False)])
def test_decode_shapes(io, N, gate):
    print(f"decode io={io} N={N} gate={gate}", flush=True)
    inp = make_decode_case(400 + N, 7, 37, N, io, gate=gate)
    d = to_dev(inp)
    state = d["state"].clone()
    y = ss.ss_state_update(state, d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d.get("z"),
                           dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    yr, sr = oracle.state_update(np64(inp["state"]), np64(inp["x"]), np64(inp["dt"]), np64(inp["A"]),
                                 np64(inp["B"]), np64(inp["C"]), D=np64(inp["D"]), z=np64(inp.get("z")),
                                 dt_bias=np64(inp["dt_bias"]))
    check_close(np64(y), yr, *TOL[io], "decode y")
    check_close(np64(state), sr, *TOL_STATE, "decode state")


@pytest.mark.parametrize("form", ["rows32", "rows32w8", "rows64"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 9, 12, 16, 17])
def test_few_row_forms_state_dims(N, io, form, monkeypatch):
    """The forms for few rows (rows of 32 and 64 lanes: the chunk scan over 2
    and 4 DPP rows, B/C staged in 8- and 4-coordinate groups) at every
    instantiated state width, a ragged channel count (21: partial blocks) and
    a ragged tail over several chunks of 512 and 1024 tokens; N = 17 is past
    their range and takes the plain scan."""
    force_scan_kernel(monkeypatch, form)
    print(f"few-row form {form} io={io} N={N}", flush=True)
    inp = make_case(330 + N, 2, 21, N, 2777, io, gate=N % 2 == 0, h0=N % 3 != 0)
    compare_full(inp, what=f"{form} {io} N={N}")
