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
