"""Shared test plumbing: run the oracle on (sampled rows of) a case and
compare GPU outputs with it at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# |gpu - oracle| <= atol + rtol * |oracle|, elementwise.
# fp32 I/O: the stated 1e-4 relative / 1e-5 absolute.
# bf16 I/O: the stated 2e-2 relative; the absolute term covers y near 0 where
# the relative bar is empty: fp32 accumulation of the ~N+2 terms of y (each
# |term| <~ 10 here) errs by <~ 1e-5, and rounding y to bf16 adds <= 2^-9 |y|.
TOL = {"f32": (1e-4, 1e-5), "bf16": (2e-2, 1e-4)}
# h_last is float32 for every I/O type; the state is fp32 end to end, so it is
# held to the fp32 bar.
TOL_STATE = (1e-4, 1e-5)


def io_name(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def oracle_scan_full(inp, dt_softplus=True, threads=None):
    return oracle.scan(np64(inp["x"]), np64(inp["dt"]), np64(inp["A"]), np64(inp["B"]), np64(inp["C"]),
                       D=np64(inp["D"]), z=np64(inp.get("z")), dt_bias=np64(inp["dt_bias"]),
                       h0=np64(inp.get("h0")), reset=None if inp.get("reset") is None else inp["reset"].numpy(),
                       dt_softplus=dt_softplus, threads=threads)


def oracle_scan_rows(inp, rows, dt_softplus=True):
    """Oracle y [len(rows), L] and h_last [len(rows), N] for the (b, c) rows,
    computed row by row from the rows' own slices of the inputs."""
    ys, hs = [], []
    for b, c in rows:
        sl = lambda t: None if t is None else t[b:b + 1, c:c + 1]
        y, h = oracle.scan(np64(sl(inp["x"])), np64(sl(inp["dt"])), np64(inp["A"][c:c + 1]),
                           np64(inp["B"][b:b + 1]), np64(inp["C"][b:b + 1]), D=np64(inp["D"][c:c + 1]),
                           z=np64(sl(inp.get("z"))), dt_bias=np64(inp["dt_bias"][c:c + 1]),
                           h0=np64(sl(inp.get("h0"))),
                           reset=None if inp.get("reset") is None else inp["reset"][b:b + 1].numpy(),
                           dt_softplus=dt_softplus, threads=1)
        ys.append(y[0, 0])
        hs.append(h[0, 0])
    return np.stack(ys), np.stack(hs)


def sample_rows(batch, channels, k, seed):
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (batch - 1, channels - 1), (0, channels - 1), (batch - 1, 0)}
    while len(rows) < min(k, batch * channels):
        rows.add((int(rng.integers(batch)), int(rng.integers(channels))))
    return sorted(rows)


def check_close(gpu, ref, rtol, atol, what):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {"max_abs": 0.0}
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    bad = err > bound
    stats = {"max_abs": float(err.max()), "max_rel": float((err / np.maximum(np.abs(r), 1e-30)).max()),
             "worst_ratio": float((err / bound).max())}
    if bad.any():
        idx = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} outside |d| <= {atol} + {rtol}|ref|; "
                             f"worst at {idx}: gpu {g[idx]!r} ref {r[idx]!r}; {stats}")
    return stats


def to_dev(inp, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


# The prompt-scan kernel variants the GPU tests run: the chunked scan at 16
# and at 32 tokens per lane; its forms for few rows at 16 tokens per lane,
# rows of 32 lanes (4- and 8-wave blocks) or 64 lanes; and the row-parallel
# walk. The library picks one by shape; SS_SCAN_KERNEL,
# SS_SCAN_TOKENS_PER_LANE and SS_SCAN_FORM, read at every call, force one.
# (The few-row forms take no reset mask and N <= 16: past that, they run the
# plain chunked scan.)
_FORMS = {"rows32": "r32w4", "rows32w8": "r32w8", "rows64": "r64w4"}
SCAN_KERNELS = ["chunked", "chunked32", *_FORMS, "rows"]
RESET_SCAN_KERNELS = ["chunked", "chunked32", "rows"]


def force_scan_kernel(monkeypatch, kind):
    monkeypatch.setenv("SS_SCAN_KERNEL", "rows" if kind == "rows" else "chunked")
    monkeypatch.setenv("SS_SCAN_TOKENS_PER_LANE", "32" if kind == "chunked32" else "16")
    monkeypatch.setenv("SS_SCAN_FORM", _FORMS.get(kind, "plain"))
