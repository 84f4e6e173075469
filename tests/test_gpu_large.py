"""GPU parity at sizes past 2^31 elements per tensor: every element offset
past 2^31 needs 64-bit arithmetic in the kernels' addressing.

Shape: batch 1, channels 4100 (not a multiple of any channel block), seq
524,296 (whole 16-byte vectors, so the vectorised paths run, and a ragged last
256-token chunk): 2,149,613,600 elements in each of x, dt, z, y (4.3 GB each
in bf16). The large tensors are drawn on the device with torch's
seeded generator (standard normal, as the workloads draw them); the small ones
(A, D, dt_bias, h0, B, C, conv and projection weights) with the workloads'
recipes on the CPU. Rows are independent, so the oracle checks whole sampled
rows, among them the last channel (the largest offsets), from those rows'
own slices of the inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import s4d_real_A
from tests.helpers import TOL, TOL_STATE, check_close, np64, oracle_scan_rows

pytestmark = pytest.mark.gpu

BATCH, CHANNELS, N, L = 1, 4100, 16, 524_296
ROWS = [0, 1, 2047, 2048, 4095, 4099]


def big_normal(seed, shape):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def cpu_normal(seed, shape, mean=0.0, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g) * std + mean


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_scan_past_2_31_elements():
    assert BATCH * CHANNELS * L > 2 ** 31
    print(f"large scan {BATCH} x {CHANNELS} x {N} x {L} bf16 gate h0", flush=True)
    x, dt, z = big_normal(11, (BATCH, CHANNELS, L)), big_normal(12, (BATCH, CHANNELS, L)), big_normal(13, (BATCH, CHANNELS, L))
    Bm = cpu_normal(14, (BATCH, N, L)).to(torch.bfloat16)
    Cm = cpu_normal(15, (BATCH, N, L)).to(torch.bfloat16)
    A = s4d_real_A(CHANNELS, N)
    D = cpu_normal(16, (CHANNELS,))
    dt_bias = cpu_normal(17, (CHANNELS,), -4.0, 0.5)
    h0 = cpu_normal(18, (BATCH, CHANNELS, N), 0.0, 0.1)
    y, h = ss.ss_scan_fwd(x, dt, A.cuda(), Bm.cuda(), Cm.cuda(), D=D.cuda(), z=z, dt_bias=dt_bias.cuda(),
                          h0=h0.cuda(), dt_softplus=True)
    torch.cuda.synchronize()
    sub = {"x": x[:, ROWS].cpu(), "dt": dt[:, ROWS].cpu(), "z": z[:, ROWS].cpu(), "B": Bm, "C": Cm,
           "A": A[ROWS], "D": D[ROWS], "dt_bias": dt_bias[ROWS], "h0": h0[:, ROWS], "reset": None}
    yg, hg = y[0, ROWS].cpu(), h[0, ROWS].cpu()
    del x, dt, z, y, h
    free()
    yr, hr = oracle_scan_rows(sub, [(0, i) for i in range(len(ROWS))])
    check_close(np64(yg), yr, *TOL["bf16"], "y past 2^31")
    check_close(np64(hg), hr, *TOL_STATE, "h_last past 2^31")


def test_conv1d_silu_past_2_31_elements():
    print(f"large conv1d + SiLU {BATCH} x {CHANNELS} x {L} bf16 width 4", flush=True)
    x_pre = big_normal(21, (BATCH, CHANNELS, L))
    w = cpu_normal(22, (CHANNELS, 4), 0.0, 0.5)
    b = cpu_normal(23, (CHANNELS,), 0.0, 0.1)
    x = ss.ss_conv1d_silu(x_pre, w.cuda(), b.cuda())
    torch.cuda.synchronize()
    xs, xg = x_pre[:, ROWS].cpu(), x[0, ROWS].cpu()
    del x_pre, x
    free()
    xr = oracle.conv1d_silu(np64(xs), np64(w[ROWS]), np64(b[ROWS]))
    check_close(np64(xg), xr[0], *TOL["bf16"], "conv1d + SiLU past 2^31")


def test_dt_proj_past_2_31_outputs():
    R = 160
    print(f"large dt_proj {BATCH} x {CHANNELS} x {L} rank {R} bf16 softplus", flush=True)
    delta = big_normal(31, (BATCH, L, R)) * 0.1
    w_dt = (cpu_normal(32, (CHANNELS, R)) * 0.1).to(torch.bfloat16)
    bias = cpu_normal(33, (CHANNELS,), -4.0, 0.5)
    dt = ss.ss_dt_proj(w_dt.cuda(), delta, bias.cuda(), apply_softplus=True)
    torch.cuda.synchronize()
    assert dt.numel() > 2 ** 31
    dg = dt[0, ROWS].cpu()
    ds = delta.cpu()
    del dt, delta
    free()
    dr = oracle.dt_proj(np64(w_dt[ROWS]), np64(ds), np64(bias[ROWS]), apply_softplus=True)
    check_close(np64(dg), dr[0], *TOL["bf16"], "dt_proj past 2^31")


def test_decode_state_past_2_31_elements():
    Bn, Cn = 4096, 32776
    assert Bn * Cn * N > 2 ** 31
    print(f"large decode {Bn} x {Cn} x {N} bf16 gate, fp32 state", flush=True)
    g = torch.Generator(device="cuda").manual_seed(41)
    state = torch.randn((Bn, Cn, N), generator=g, device="cuda", dtype=torch.float32)
    x, dt, z = big_normal(42, (Bn, Cn)), big_normal(43, (Bn, Cn)), big_normal(44, (Bn, Cn))
    Bm = cpu_normal(45, (Bn, N)).to(torch.bfloat16)
    Cm = cpu_normal(46, (Bn, N)).to(torch.bfloat16)
    A = s4d_real_A(Cn, N)
    D = cpu_normal(47, (Cn,))
    dt_bias = cpu_normal(48, (Cn,), -4.0, 0.5)
    bs, cs = [0, 1, Bn - 1], [0, 17, Cn - 1]
    sub = lambda t: t[bs][:, cs].cpu()
    s_before = sub(state)
    y = ss.ss_state_update(state, x, dt, A.cuda(), Bm.cuda(), Cm.cuda(), D=D.cuda(), z=z, dt_bias=dt_bias.cuda())
    torch.cuda.synchronize()
    s_after, yg, xs, dts, zs = sub(state), sub(y), sub(x), sub(dt), sub(z)
    del state, x, dt, z, y
    free()
    yr, sr = oracle.state_update(np64(s_before), np64(xs), np64(dts), np64(A[cs]), np64(Bm[bs]), np64(Cm[bs]),
                                 D=np64(D[cs]), z=np64(zs), dt_bias=np64(dt_bias[cs]))
    check_close(np64(yg), yr, *TOL["bf16"], "decode y past 2^31")
    check_close(np64(s_after), sr, *TOL_STATE, "decode state past 2^31")


def test_every_token_states_past_2_31_elements():
    Cn, Ls = 64, 2 ** 21 + 8
    assert Cn * N * Ls > 2 ** 31
    print(f"large states {BATCH} x {Cn} x {N} x {Ls} bf16 gate h0", flush=True)
    x, dt, z = big_normal(51, (BATCH, Cn, Ls)), big_normal(52, (BATCH, Cn, Ls)), big_normal(53, (BATCH, Cn, Ls))
    Bm = cpu_normal(54, (BATCH, N, Ls)).to(torch.bfloat16)
    Cm = cpu_normal(55, (BATCH, N, Ls)).to(torch.bfloat16)
    A = s4d_real_A(Cn, N)
    D = cpu_normal(56, (Cn,))
    dt_bias = cpu_normal(57, (Cn,), -4.0, 0.5)
    h0 = cpu_normal(58, (BATCH, Cn, N), 0.0, 0.1)
    y, h, st = ss.ss_scan_fwd_states(x, dt, A.cuda(), Bm.cuda(), Cm.cuda(), D=D.cuda(), z=z, dt_bias=dt_bias.cuda(),
                                     h0=h0.cuda())
    torch.cuda.synchronize()
    assert st.numel() > 2 ** 31
    rows = [0, Cn - 1]
    stg, yg, hg = st[0, rows].cpu(), y[0, rows].cpu(), h[0, rows].cpu()
    xs, dts, zs = x[:, rows].cpu(), dt[:, rows].cpu(), z[:, rows].cpu()
    del x, dt, z, y, h, st
    free()
    yr, hr, sr = oracle.scan(np64(xs), np64(dts), np64(A[rows]), np64(Bm), np64(Cm), D=np64(D[rows]), z=np64(zs),
                             dt_bias=np64(dt_bias[rows]), h0=np64(h0[:, rows]), return_states=True)
    check_close(np64(yg), yr[0], *TOL["bf16"], "states-scan y past 2^31")
    check_close(np64(hg), hr[0], *TOL_STATE, "states-scan h_last past 2^31")
    check_close(np64(stg), sr[0].transpose(0, 2, 1), *TOL_STATE, "every-token states past 2^31")


@pytest.mark.parametrize("per_state", [False, True], ids=["summed", "per_state"])
def test_effective_attention_past_2_31_elements(per_state):
    Cn, La, W = (2, 8200, 256) if per_state else (32, 8200, 256)
    assert Cn * (N if per_state else 1) * La * La > 2 ** 31
    print(f"large effective attention {BATCH} x {Cn} x {N} x {La} bf16 per_state={per_state}", flush=True)
    dt = big_normal(61, (BATCH, Cn, La))
    Bm = cpu_normal(62, (BATCH, N, La)).to(torch.bfloat16)
    Cm = cpu_normal(63, (BATCH, N, La)).to(torch.bfloat16)
    A = s4d_real_A(Cn, N)
    dt_bias = cpu_normal(64, (Cn,), -4.0, 0.5)
    M = ss.ss_effective_attention(dt, A.cuda(), Bm.cuda(), Cm.cuda(), dt_bias.cuda(), per_state_coord=per_state)
    torch.cuda.synchronize()
    assert M.numel() > 2 ** 31
    c = Cn - 1
    head, tail = slice(0, W), slice(La - W, La)
    Mc = M[0, c]
    blocks = {k: Mc[..., r, s].cpu() for k, (r, s) in
              {"head": (head, head), "tail": (tail, tail), "corner": (tail, head), "upper": (head, tail)}.items()}
    dts = dt[0, c].cpu()
    del M, Mc, dt
    free()
    # M[i, j] involves only the tokens j .. i, so a diagonal block is the
    # oracle's matrix of that window of tokens
    for name, win in (("head", head), ("tail", tail)):
        d = np64(dts[win]).reshape(1, 1, W)
        kw = dict(dt_bias=np64(dt_bias[c:c + 1]), per_state_coord=per_state)
        ref = oracle.effective_attention(d, np64(A[c:c + 1]), np64(Bm[:, :, win]), np64(Cm[:, :, win]), **kw)[0, 0]
        scale = np.abs(oracle.effective_attention(d, np64(A[c:c + 1]), np.abs(np64(Bm[:, :, win])),
                                                  np.abs(np64(Cm[:, :, win])), **kw)[0, 0])
        g = np64(blocks[name])
        err = np.abs(g - ref)
        bound = 1e-4 * np.abs(ref) + 1e-5 + (W + 2 * N) * 2.0 ** -24 * scale
        assert np.isfinite(g).all() and (err <= bound).all(), f"{name} block: worst {(err - bound).max()}"
    # above the diagonal: exact zeros; far below it the decay over ~8000 tokens
    # is below fp32's range (the oracle's value there is under 1e-30)
    assert (blocks["upper"] == 0).all()
    assert (blocks["corner"].abs() <= 1e-30).all()


def test_gated_scan_past_2_31_elements():
    Bh, Lg, dk, dv = 128, 131_080, 128, 64
    assert Bh * Lg * dk > 2 ** 31
    print(f"large gated scan {Bh} x {Lg} x {dk} x {dv} bf16", flush=True)
    q = big_normal(71, (Bh, Lg, dk)) * dk ** -0.5
    k = big_normal(72, (Bh, Lg, dk)) * dk ** -0.5
    v = big_normal(73, (Bh, Lg, dv))
    g = torch.Generator(device="cuda").manual_seed(74)
    gamma = torch.rand((Bh, Lg), generator=g, device="cuda") * 0.1 + 0.9
    s0 = cpu_normal(75, (Bh, dk, dv))
    y, fs = ss.ss_gated_scan(q, k, v, gamma, s0.cuda())
    torch.cuda.synchronize()
    h = Bh - 1
    qs, ks, vs, gs = q[h:].cpu(), k[h:].cpu(), v[h:].cpu(), gamma[h:].cpu()
    yg, fg = y[h:].cpu(), fs[h:].cpu()
    del q, k, v, gamma, y, fs
    free()
    args = [np64(t) for t in (qs, ks, vs, gs)]
    yr, fr = oracle.gated_scan(*args, s0=np64(s0[h:]))
    ya, fa = oracle.gated_scan(*[np.abs(a) for a in args], s0=np.abs(np64(s0[h:])))
    # y in bf16, the final state in fp32: the gated tests' bound, rtol |r| + atol + 2^-19 S
    for got, ref, ref_abs, (rtol, atol), what in ((yg, yr, ya, TOL["bf16"], "y"),
                                                  (fg, fr, fa, TOL["f32"], "final state")):
        gg = np64(got)
        err = np.abs(gg - ref)
        bound = rtol * np.abs(ref) + atol + 2.0 ** -19 * np.abs(ref_abs)
        assert np.isfinite(gg).all() and (err <= bound).all(), f"gated {what} past 2^31: worst {(err - bound).max()}"
