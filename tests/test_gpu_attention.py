"""GPU parity of ss_effective_attention (TransformerLens "ssm_mixer" page,
compute_effective_attention) against the fp64 oracle on the same seeded
inputs.

Tolerance, from the arithmetic: an element is a sum over n of C B times a
product of (i - j) factors exp(A dt_k), each rounded to fp32; the kernel
extends the product one factor per row, so the relative error of a term
grows by about one rounding per factor, and the sum adds N more. With the
absolute sum of the terms (the oracle on |B|, |C|) as the scale, the bar is

    |gpu - oracle| <= 1e-4 |oracle| + 1e-5 + (L + 2 N) 2^-24 * absolute sum

(the fp32 pair of the selective scan, plus the chain-length term that only
matters where the terms cancel)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import make_case
from tests.helpers import np64

pytestmark = pytest.mark.gpu


def oracle_attn(inp, softplus=True, include_dt=False, per_state=False, rows=None):
    """Oracle M and its absolute-sum scale, for all channels or a channel subset."""
    dt, A, bias = np64(inp["dt"]), np64(inp["A"]), np64(inp["dt_bias"])
    if rows is not None:
        dt, A, bias = dt[:, rows], A[rows], bias[rows]
    B, C = np64(inp["B"]), np64(inp["C"])
    kw = dict(dt_bias=bias, dt_softplus=softplus, include_dt_scaling=include_dt, per_state_coord=per_state)
    M = oracle.effective_attention(dt, A, B, C, **kw)
    Ma = oracle.effective_attention(dt, A, np.abs(B), np.abs(C), **kw)
    return M, np.abs(Ma)


def check(got, ref, scale, L, N, what):
    g = np64(got)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = 1e-4 * np.abs(ref) + 1e-5 + (L + 2 * N) * 2.0 ** -24 * scale
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; worst at {i}: "
                             f"gpu {g[i]!r} oracle {ref[i]!r} scale {scale[i]!r}")


def run(d, **kw):
    return ss.ss_effective_attention(d["dt"], d["A"], d["B"], d["C"], d["dt_bias"], **kw)


def to_dev(inp):
    return {k: None if v is None else v.cuda() for k, v in inp.items()}


CASES = [
    # io, batch, channels, N, L, softplus, include_dt, per_state
    ("f32", 1, 3, 4, 17, True, False, False),
    ("bf16", 2, 5, 16, 130, True, True, False),
    ("f32", 1, 2, 16, 300, True, False, False),
    ("bf16", 1, 3, 9, 64, True, True, True),
    ("f32", 2, 2, 33, 100, False, False, True),
    ("bf16", 1, 2, 64, 257, True, True, False),
    ("f32", 1, 2, 8, 513, True, True, False),
    ("bf16", 3, 1, 16, 1, True, False, False),
    ("bf16", 1, 2, 16, 512, True, True, False),   # the tiled form's longest sequence (32 row tiles)
    ("f32", 2, 3, 12, 48, False, False, False),   # three whole tiles, softplus off
]


@pytest.mark.parametrize("io,batch,channels,N,L,softplus,include_dt,per_state", CASES,
                         ids=[f"{c[0]}-b{c[1]}-c{c[2]}-N{c[3]}-L{c[4]}-sp{int(c[5])}-dt{int(c[6])}-ps{int(c[7])}"
                              for c in CASES])
def test_attention_parity(io, batch, channels, N, L, softplus, include_dt, per_state):
    print(f"attention io={io} b={batch} c={channels} N={N} L={L} sp={softplus} dt={include_dt} ps={per_state}",
          flush=True)
    inp = make_case(1200 + L + N, batch, channels, N, L, io, gate=False, h0=False)
    if not softplus:
        # without softplus the step size is dt + dt_bias itself; a bias of 4
        # keeps it positive (a decaying product), as a step size is
        inp["dt_bias"] = torch.full_like(inp["dt_bias"], 4.0)
    d = to_dev(inp)
    M = run(d, dt_softplus=softplus, include_dt_scaling=include_dt, per_state_coord=per_state)
    torch.cuda.synchronize()
    ref, scale = oracle_attn(inp, softplus, include_dt, per_state)
    check(M, ref, scale, L, N, "M")
    upper = np.triu(np.ones((L, L), dtype=bool), 1)
    assert np.all(np64(M)[..., upper] == 0.0), "nonzero above the diagonal"


def test_attention_reconstructs_gpu_scan():
    """The page's reconstruction form against the library's own scan:
    sum_j M[c, i, j] x[c, j] + D[c] x[c, i] is ss_scan_fwd's output with no
    gate and a zero state (fp32 I/O, the fp32 bar on the absolute sum of
    the products)."""
    print("attention reconstruction", flush=True)
    inp = make_case(1290, 2, 6, 16, 200, "f32", gate=False, h0=False)
    d = to_dev(inp)
    M = run(d, include_dt_scaling=True)
    y, _ = ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"])
    y_rec = torch.einsum("bcij,bcj->bci", M.double(), d["x"].double()) + d["D"].double()[None, :, None] * d["x"]
    scale = torch.einsum("bcij,bcj->bci", M.double().abs(), d["x"].double().abs()) + (d["D"].abs()[None, :, None]
                                                                                     * d["x"].abs())
    torch.cuda.synchronize()
    err = (y.double() - y_rec).abs()
    assert bool((err <= 1e-4 * y_rec.abs() + 1e-5 + 1e-5 * scale).all()), float(err.max())


def test_attention_full_size_sampled():
    """Mamba-130M-shaped layer at a short sequence: batch 1, channels 1536,
    state_dim 16, seq 256, bf16 inputs (403 MB of fp32 output); sampled
    channels against the oracle on their own slices."""
    print("attention full size 1x1536x16x256", flush=True)
    inp = make_case(1291, 1, 1536, 16, 256, "bf16", gate=False, h0=False)
    d = to_dev(inp)
    M = run(d)
    M2 = run(d)
    torch.cuda.synchronize()
    assert torch.equal(M, M2), "not bitwise reproducible"
    rows = [0, 1, 777, 1535]
    ref, scale = oracle_attn(inp, rows=rows)
    check(M[:, rows], ref, scale, 256, 16, "M sampled channels")


def test_attention_errors():
    inp = to_dev(make_case(1292, 1, 2, 16, 32, "f32", gate=False, h0=False))
    bad_A = torch.zeros(2, 65, device="cuda")
    B65 = torch.zeros(1, 65, 32, device="cuda")
    with pytest.raises(ss.SSError) as e:
        ss.ss_effective_attention(inp["dt"], bad_A, B65, B65)
    assert e.value.code == 4
    big = torch.empty(1, 2, 32, 32, device="cuda")        # the output, with dt stored inside it
    dt_view = big.view(-1)[:64].view(1, 2, 32)
    dt_view.copy_(inp["dt"])
    with pytest.raises(ss.SSError) as e:
        ss.ss_effective_attention(dt_view, inp["A"], inp["B"], inp["C"], inp["dt_bias"], out=big)
    assert e.value.code == 5


def test_attention_edges():
    """Zero-size calls are no-ops; one channel of one token is C . B."""
    print("attention edges", flush=True)
    inp = to_dev(make_case(1293, 1, 3, 16, 0, "f32", gate=False, h0=False))
    assert run(inp).shape == (1, 3, 0, 0)
    inp = make_case(1294, 2, 1, 5, 1, "f32", gate=False, h0=False)
    M = run(to_dev(inp))
    torch.cuda.synchronize()
    ref = (np64(inp["C"])[:, :, 0] * np64(inp["B"])[:, :, 0]).sum(1)
    assert np.allclose(np64(M)[:, 0, 0, 0], ref, rtol=1e-5, atol=1e-6)
