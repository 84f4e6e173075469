"""MI355X (gfx950) Mamba-1 S6 selective scan.

The compute lives in the HIP library ``libssscan.so`` (C ABI declared in
``include/ss_scan.h``); this package is its thin Python binding. The two
entry points keep the C names and the argument order of the kernel calls on
the nnterp "selective_scan" page:

    ss_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None,
                reset=None, dt_softplus=True) -> (y, h_last)
    ss_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                    dt_softplus=True) -> y          (state updated in place)

and the scan that also returns the state after every token, or after one
selected token:

    ss_scan_fwd_states(..., time_step=None) -> (y, h_last, states)

and the scalar-gated state scan of the "Mamba 2 Gated State Scan" page:

    ss_gated_scan(q, k, v, gamma, s0=None) -> (y, final_state)

the producers of the scan's inputs (the causal conv1d + SiLU that makes x,
and the dt_proj projection that makes dt):

    ss_conv1d_silu(x_pre, conv_w, conv_b=None, reset=None) -> x
    ss_dt_proj(w_dt, delta, dt_bias=None, apply_softplus=False) -> dt

and the scan with the conv1d + SiLU fused in (x made in registers from
x_pre, never written to memory):

    ss_scan_fwd_conv(x_pre, dt, A, B, C, conv_w, conv_b=None, D=None, ...) -> (y, h_last)

and the scan's effective attention of the TransformerLens "ssm_mixer" page:

    ss_effective_attention(dt, A, B, C, dt_bias=None, include_dt_scaling=False,
                           per_state_coord=False) -> M

Arguments are torch tensors on the GPU: the binding checks them, allocates
the outputs with torch and passes raw device pointers plus the current HIP
stream. Every step of the computation runs in the library's kernels; there is
no other implementation to fall back to, and a missing library is an error.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    SSError,
    abi_version,
    ss_conv1d_silu,
    ss_dt_proj,
    ss_effective_attention,
    ss_gated_scan,
    library_path,
    load_library,
    ss_scan_fwd,
    ss_scan_fwd_conv,
    ss_scan_fwd_states,
    ss_state_update,
    status_str,
)
