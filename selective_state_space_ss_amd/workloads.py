"""Seeded synthetic inputs for the selective-scan workloads.

This module only draws random numbers and lays them out; it holds none of the
scan's arithmetic, so both the HIP path and the CPU oracle can be fed from it.

The five workloads are Mamba-1 S6 selective-scan calls at the shapes the method
is used at (nnterp "selective_scan" page, class docstring: channel-first kernel
tensors x, dt [batch, channels, seq], B, C [batch, state_dim, seq], A
[channels, state_dim], a decode step drops the seq axis; mixle
"selective_scan" page, module doc: S4D-real initialisation of A).

Recipe (all draws fp32 from one ``torch.Generator`` seeded per workload, in
the fixed order x, dt_raw, z, B, C, D, dt_bias, h0/state, reset; draws a
workload does not use are skipped; ``N(mu, s)`` means ``mu + s * randn``;
bf16 tensors are the fp32 draws rounded to nearest-even by ``Tensor.to``):

* ``A[c, n] = -(n + 1)`` (S4D-real); parity cases may instead draw a
  different A for every (c, n) (``learned_like_A``).
* ``x, B, C, z, D ~ N(0, 1)``; ``dt_raw ~ N(0, 1)``.
* ``dt_bias ~ N(-4, 0.5)`` per channel, except ``mamba130m`` where
  ``dt_bias = softplus^-1(u)``, ``u = exp(Uniform(ln 1e-3, ln 0.1))``.
* ``mamba2p8b``: ``h0 ~ N(0, 0.1)``; ``decode``: cached ``state ~ N(0, 1)``.
* ``packed_reset``: ``reset[b, 0] = 1`` and ``reset[b, t >= 1]`` i.i.d.
  Bernoulli(1/512), i.e. geometric document lengths with mean 512 (the last
  document of a row is cut by the row's end).

Scalar-gated state scan cases ("Mamba 2 Gated State Scan" page: q, k
[batch, seq, dk], v [batch, seq, dv], gamma [batch, seq] in [0, 1]), drawn
in the order q, k, v, gamma, zero mask, s0: ``q, k ~ N(0, dk^-1/2)``,
``v ~ N(0, 1)``; ``gamma ~ Uniform(0.9, 1)`` ("decay"), ``Uniform(0, 1)``
("uniform"), or exactly 1 or 0; with ``zero_rate`` each gamma is also set to
0 with that probability (a state cleared at that token); ``s0 ~ N(0, 1)``.

Input-side producer cases (the conv1d + SiLU that makes x, the dt_proj
projection that makes dt), drawn in the order x_pre, conv_w, conv_b, w_dt,
delta, dt_bias, reset: ``x_pre ~ N(0, 1)``, ``conv_w ~ N(0, W^-1/2)``,
``conv_b ~ N(0, 0.1)``, ``w_dt ~ N(0, R^-1/2)``, ``delta ~ N(0, 1)``
(token-major [batch, L, R]), ``dt_bias ~ N(-4, 0.5)``, and the packed-reset
mask recipe above when a mean document length is given.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    channels: int
    state_dim: int
    seqlen: int           # 0 marks the single-token decode step (no seq axis)
    io_dtype: str         # "f32" or "bf16": dtype of x, dt, z, B, C and y
    gate: bool            # silu(z) gate on
    h0: Optional[float]   # std of the random initial / cached state, or None
    reset_mean_doc: Optional[int]  # mean document length of the reset mask
    dt_bias: str          # "normal" (N(-4, 0.5)) or "loguniform"
    seed: int
    note: str

    @property
    def decode(self) -> bool:
        return self.seqlen == 0

    @property
    def channel_tokens(self) -> int:
        return self.batch * self.channels * max(self.seqlen, 1)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1, 8, 4, 64, "f32", False, None, None, "normal", 1001,
                 "tiny S6 prompt scan, fp32, zero initial state, no gate"),
        Workload("mamba130m", 4, 1536, 16, 2048, "bf16", True, None, None, "loguniform", 1002,
                 "Mamba-130M-shaped layer (d_inner 1536), gated"),
        Workload("mamba2p8b", 8, 5120, 16, 2048, "bf16", True, 0.1, None, "normal", 1003,
                 "Mamba-2.8B-shaped layer (d_inner 5120), gated, random h0"),
        Workload("packed_reset", 4, 2048, 16, 8192, "bf16", False, None, 512, "normal", 1004,
                 "packed sequences with hard reset at document starts"),
        Workload("decode", 256, 5120, 16, 0, "bf16", True, 1.0, None, "normal", 1005,
                 "single-token decode step, cached fp32 state updated in place"),
    ]
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def io_torch_dtype(w: Workload) -> torch.dtype:
    return _TORCH_DTYPE[w.io_dtype]


def _normal(gen: torch.Generator, shape, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32)
    t.normal_(generator=gen)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def s4d_real_A(channels: int, state_dim: int) -> torch.Tensor:
    """A[c, n] = -(n + 1), the S4D-real initialisation."""
    row = -torch.arange(1, state_dim + 1, dtype=torch.float32)
    return row.unsqueeze(0).expand(channels, state_dim).contiguous()


def learned_like_A(seed: int, channels: int, state_dim: int) -> torch.Tensor:
    """A different for every (c, n), as a trained model's A = -exp(A_log)
    is: ``A = -exp(N(0.5, 1))`` (mostly 0.2 .. 12, tails past 50), with about
    5 % of the entries exactly 0 (no decay) and 2 % at -5000 (the state
    forgets within a token). Its own generator, seeded with ``seed``."""
    gen = torch.Generator().manual_seed(seed)
    A = -torch.exp(_normal(gen, (channels, state_dim), 0.5, 1.0))
    u = torch.rand((channels, state_dim), generator=gen)
    A = torch.where(u < 0.05, torch.zeros_like(A), A)
    return torch.where((u >= 0.05) & (u < 0.07), torch.full_like(A, -5000.0), A).contiguous()


def reset_mask(gen: torch.Generator, batch: int, seqlen: int, mean_doc: int) -> torch.Tensor:
    """uint8 [batch, seqlen]; 1 marks the first token of a document."""
    u = torch.rand((batch, seqlen), generator=gen)
    m = (u < (1.0 / mean_doc)).to(torch.uint8)
    if seqlen > 0:
        m[:, 0] = 1
    return m


def make_inputs(w: Workload | str, seed: Optional[int] = None, *, batch: Optional[int] = None,
                channels: Optional[int] = None, seqlen: Optional[int] = None,
                state_dim: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one workload's inputs as CPU tensors.

    Shape overrides keep the workload's distributions at another size (used
    for small parity cases). Keys: x, dt, z, B, C, A, D, dt_bias, h0 (prompt)
    or state (decode), reset; absent inputs are None.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    Bn = w.batch if batch is None else batch
    Cn = w.channels if channels is None else channels
    L = w.seqlen if seqlen is None else seqlen
    N = w.state_dim if state_dim is None else state_dim
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    io = io_torch_dtype(w)
    tok = (Bn, Cn) if w.decode else (Bn, Cn, L)
    bc = (Bn, N) if w.decode else (Bn, N, L)

    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal(gen, tok).to(io)
    out["dt"] = _normal(gen, tok).to(io)
    out["z"] = _normal(gen, tok).to(io) if w.gate else None
    out["B"] = _normal(gen, bc).to(io)
    out["C"] = _normal(gen, bc).to(io)
    out["D"] = _normal(gen, (Cn,))
    if w.dt_bias == "loguniform":
        u = torch.empty((Cn,), dtype=torch.float32).uniform_(math.log(1e-3), math.log(0.1), generator=gen).exp()
        # inverse of softplus: log(exp(u) - 1), evaluated in float64 for the small u
        out["dt_bias"] = torch.log(torch.expm1(u.double())).float()
    else:
        out["dt_bias"] = _normal(gen, (Cn,), -4.0, 0.5)
    h_shape = (Bn, Cn, N)
    if w.decode:
        out["state"] = _normal(gen, h_shape, 0.0, w.h0 if w.h0 is not None else 1.0)
        out["h0"] = None
    else:
        out["h0"] = _normal(gen, h_shape, 0.0, w.h0) if w.h0 is not None else None
    out["reset"] = (reset_mask(gen, Bn, L, w.reset_mean_doc)
                    if (w.reset_mean_doc is not None and not w.decode) else None)
    out["A"] = s4d_real_A(Cn, N)
    return out


def algorithmic_bytes(w: Workload) -> int:
    """Bytes the method must move once: every input read once, every output
    written once (the per-token state is never materialised)."""
    s = 2 if w.io_dtype == "bf16" else 4
    Bn, Cn, N = w.batch, w.channels, w.state_dim
    L = max(w.seqlen, 1)
    tok = Bn * Cn * L
    n = 0
    n += tok * s * (2 + (1 if w.gate else 0))   # x, dt (, z)
    n += tok * s                                # y
    n += 2 * Bn * N * L * s                     # B, C
    n += Cn * N * 4 + 2 * Cn * 4                # A, D, dt_bias
    if w.decode:
        n += 2 * Bn * Cn * N * 4                # state read + write
    else:
        if w.h0 is not None:
            n += Bn * Cn * N * 4                # h0
        n += Bn * Cn * N * 4                    # h_last
        if w.reset_mean_doc is not None:
            n += Bn * L                         # reset mask
    return n


def make_case(seed: int, batch: int, channels: int, state_dim: int, seqlen: int, io_dtype: str = "bf16",
              gate: bool = True, h0: bool = True, reset_mean_doc: Optional[int] = None,
              dt_bias: str = "normal", a_init: str = "s4d") -> Dict[str, Optional[torch.Tensor]]:
    """An arbitrary-shape prompt case with the workloads' distributions
    (h0 ~ N(0, 0.1) when requested); seqlen == 0 is allowed. Same key set as
    make_inputs. a_init="learned" replaces the S4D-real A by
    learned_like_A(seed + 7919, ...)."""
    w = Workload("case", batch, channels, state_dim, max(seqlen, 1), io_dtype, gate, 0.1 if h0 else None,
                 reset_mean_doc, dt_bias, seed, "parity case")
    out = make_inputs(w, seqlen=seqlen)
    if a_init == "learned":
        out["A"] = learned_like_A(seed + 7919, channels, state_dim)
    elif a_init != "s4d":
        raise ValueError(f"a_init: {a_init!r}")
    return out


def make_decode_case(seed: int, batch: int, channels: int, state_dim: int, io_dtype: str = "bf16",
                     gate: bool = True, a_init: str = "s4d") -> Dict[str, Optional[torch.Tensor]]:
    """An arbitrary-shape decode-step case with the decode workload's
    distributions (a_init as for make_case)."""
    w = Workload("decode_case", batch, channels, state_dim, 0, io_dtype, gate, 1.0, None, "normal", seed,
                 "decode parity case")
    out = make_inputs(w)
    if a_init == "learned":
        out["A"] = learned_like_A(seed + 7919, channels, state_dim)
    elif a_init != "s4d":
        raise ValueError(f"a_init: {a_init!r}")
    return out


def make_gated_case(seed: int, batch: int, seqlen: int, dk: int, dv: int, io_dtype: str = "bf16",
                    gamma: str = "decay", zero_rate: float = 0.0, s0: bool = False,
                    state_dtype: Optional[str] = None, device: str = "cpu") -> Dict[str, Optional[torch.Tensor]]:
    """A scalar-gated state-scan case (recipe in the module docstring): keys
    q, k, v (io_dtype), gamma (fp32) and s0 (state_dtype, default io_dtype,
    or None)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    io = _TORCH_DTYPE[io_dtype]
    sdt = io if state_dtype is None else _TORCH_DTYPE[state_dtype]
    q = _normal(gen, (batch, seqlen, dk), std=dk ** -0.5)
    k = _normal(gen, (batch, seqlen, dk), std=dk ** -0.5)
    v = _normal(gen, (batch, seqlen, dv))
    if gamma == "decay":
        g = 0.9 + 0.1 * torch.rand((batch, seqlen), generator=gen)
    elif gamma == "uniform":
        g = torch.rand((batch, seqlen), generator=gen)
    elif gamma in ("one", "zero"):
        g = torch.full((batch, seqlen), 1.0 if gamma == "one" else 0.0)
    else:
        raise ValueError(f"unknown gamma recipe {gamma!r}")
    if zero_rate > 0.0:
        g = torch.where(torch.rand((batch, seqlen), generator=gen) < zero_rate, torch.zeros_like(g), g)
    st = _normal(gen, (batch, dk, dv)) if s0 else None
    out = {"q": q.to(io), "k": k.to(io), "v": v.to(io), "gamma": g.to(torch.float32),
           "s0": None if st is None else st.to(sdt)}
    return {key: None if t is None else t.to(device) for key, t in out.items()}


def make_producer_case(seed: int, batch: int, channels: int, seqlen: int, width: int = 4, rank: int = 160,
                       io_dtype: str = "bf16", reset_mean_doc: Optional[int] = None,
                       device: str = "cpu") -> Dict[str, Optional[torch.Tensor]]:
    """A producer case (recipe in the module docstring): keys x_pre, delta,
    w_dt (io_dtype), conv_w, conv_b, dt_bias (fp32), reset (uint8 or None)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    io = _TORCH_DTYPE[io_dtype]
    x_pre = _normal(gen, (batch, channels, seqlen))
    conv_w = _normal(gen, (channels, width), std=width ** -0.5)
    conv_b = _normal(gen, (channels,), std=0.1)
    w_dt = _normal(gen, (channels, rank), std=rank ** -0.5)
    delta = _normal(gen, (batch, seqlen, rank))
    dt_bias = _normal(gen, (channels,), mean=-4.0, std=0.5)
    reset = reset_mask(gen, batch, seqlen, reset_mean_doc) if reset_mean_doc is not None else None
    out = {"x_pre": x_pre.to(io), "conv_w": conv_w, "conv_b": conv_b, "w_dt": w_dt.to(io), "delta": delta.to(io),
           "dt_bias": dt_bias, "reset": reset}
    return {k: None if t is None else t.to(device) for k, t in out.items()}
