"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd._binding import ScanArgs, UpdateArgs, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss_scan.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIAS, HIP, ALIGN = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ss_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ss.library_path()):
        from selective_state_space_ss_amd.build import build
        build()
    return load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == ["ss_abi_version", "ss_conv1d_silu", "ss_dt_proj", "ss_effective_attention",
                                    "ss_gated_scan", "ss_scan_fwd", "ss_scan_fwd_conv", "ss_scan_fwd_states",
                                    "ss_scan_fwd_timed", "ss_state_update", "ss_state_update_timed",
                                    "ss_status_str"]


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ss.library_path()], stdout=subprocess.PIPE, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for fn in declared_functions():
        assert fn in exported, fn
        assert hasattr(lib, fn)


def test_status_strings_and_version(lib):
    assert ss.abi_version() == 9
    for code in range(8):
        assert ss.status_str(code).startswith("SS_")
    assert "unknown" in ss.status_str(99)


# Fake, well-aligned, disjoint "device" addresses: validation never dereferences them.
MB = 1 << 20


def scan_args(batch=2, channels=8, N=16, L=64, io=1, x=1 * MB, dt=2 * MB, A=3 * MB, B=4 * MB, C=5 * MB,
              D=None, z=None, bias=None, h0=None, reset=None, y=6 * MB, h_last=None):
    return ScanArgs(batch=batch, channels=channels, state_dim=N, seqlen=L, io_dtype=io, x=x, dt=dt, z=z, B=B, C=C,
                    A=A, D=D, dt_bias=bias, h0=h0, reset=reset, dt_softplus=1, y=y, h_last=h_last)


def scan_call(lib, **kw):
    return lib.ss_scan_fwd(ctypes.byref(scan_args(**kw)), None)


def upd_call(lib, batch=2, channels=8, N=16, io=1, state=1 * MB, x=2 * MB, dt=3 * MB, A=4 * MB, B=5 * MB, C=6 * MB,
             D=None, z=None, bias=None, y=7 * MB):
    a = UpdateArgs(batch=batch, channels=channels, state_dim=N, io_dtype=io, state=state, x=x, dt=dt, z=z, B=B, C=C,
                   A=A, D=D, dt_bias=bias, dt_softplus=1, y=y)
    return lib.ss_state_update(ctypes.byref(a), None)


def conv_scan_call(lib, w=9 * MB, b=None, width=4, **kw):
    return lib.ss_scan_fwd_conv(ctypes.byref(scan_args(**kw)), w, b, width, None)


def test_scan_conv_validation(lib):
    assert conv_scan_call(lib, width=0) == UNSUP
    assert conv_scan_call(lib, width=9) == UNSUP
    assert conv_scan_call(lib, w=None) == NULL
    assert conv_scan_call(lib, w=9 * MB + 2) == ALIGN
    assert conv_scan_call(lib, b=10 * MB + 1) == ALIGN
    assert conv_scan_call(lib, w=6 * MB) == ALIAS                      # weights over y
    assert conv_scan_call(lib, b=7 * MB, h_last=7 * MB) == ALIAS        # bias over h_last
    assert conv_scan_call(lib, x=None) == NULL                          # x_pre is the scan's x
    assert conv_scan_call(lib, io=4) == DTYPE
    assert conv_scan_call(lib, batch=0, w=None) == OK                   # an empty problem is a no-op
    assert lib.ss_scan_fwd_conv(None, 9 * MB, None, 4, None) == NULL


def test_null_argument_structs(lib):
    assert lib.ss_scan_fwd(None, None) == NULL
    assert lib.ss_scan_fwd_states(None, 8 * MB, -1, None) == NULL
    assert lib.ss_state_update(None, None) == NULL
    assert lib.ss_scan_fwd_timed(None, None, None, None) == NULL
    assert lib.ss_state_update_timed(None, None, None, None) == NULL


def test_timed_calls_validate_as_the_untimed_ones(lib):
    """The timed entry points run the same validation (events NULL: nothing
    to record, and no device is touched on these paths)."""
    def timed_scan(**kw):
        return lib.ss_scan_fwd_timed(ctypes.byref(scan_args(**kw)), None, None, None)

    def timed_upd(**kw):
        a = UpdateArgs(batch=kw.get("batch", 2), channels=8, state_dim=kw.get("N", 16), io_dtype=kw.get("io", 1),
                       state=kw.get("state", 1 * MB), x=2 * MB, dt=3 * MB, z=None, B=5 * MB, C=6 * MB, A=4 * MB,
                       D=None, dt_bias=None, dt_softplus=1, y=kw.get("y", 7 * MB))
        return lib.ss_state_update_timed(ctypes.byref(a), None, None, None)

    for kw in (dict(io=2), dict(batch=-1), dict(N=65), dict(x=None), dict(y=1 * MB), dict(batch=0)):
        assert timed_scan(**kw) == scan_call(lib, **kw), kw
    for kw in (dict(io=7), dict(N=65), dict(state=None), dict(y=2 * MB), dict(batch=0)):
        assert timed_upd(**kw) == upd_call(lib, **kw), kw


def test_struct_layout_matches_header(tmp_path):
    """The ctypes mirrors of ss_scan_args and ss_update_args have the C
    compiler's size and field offsets."""
    fields = {"ss_scan_args": ScanArgs, "ss_update_args": UpdateArgs}
    body = []
    for cname, py in fields.items():
        body.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            body.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "ss_scan.h"\nint main(void){' + "".join(body) +
                   "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True, check=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_scan_validation(lib):
    assert scan_call(lib, io=2) == DTYPE
    assert scan_call(lib, batch=-1) == SHAPE
    assert scan_call(lib, L=-5) == SHAPE
    assert scan_call(lib, N=0) == UNSUP
    assert scan_call(lib, N=65) == UNSUP
    assert scan_call(lib, x=None) == NULL
    assert scan_call(lib, y=None) == NULL
    assert scan_call(lib, A=None) == NULL
    assert scan_call(lib, x=1 * MB + 1) == ALIGN          # bf16 needs 2-byte alignment
    assert scan_call(lib, io=0, y=6 * MB + 2) == ALIGN    # fp32 needs 4-byte alignment
    assert scan_call(lib, y=1 * MB) == ALIAS               # y over x
    assert scan_call(lib, y=1 * MB + 128) == ALIAS         # partial overlap
    assert scan_call(lib, h0=7 * MB, h_last=7 * MB + 64) == ALIAS
    assert scan_call(lib, h_last=4 * MB) == ALIAS          # h_last over B
    assert scan_call(lib, batch=1 << 40, channels=1 << 40) == SHAPE
    # empty problems are valid no-ops and never reach the device
    assert scan_call(lib, batch=0) == OK
    assert scan_call(lib, channels=0, x=None, dt=None, B=None, C=None, y=None) == OK


def states_call(lib, states=8 * MB, time_step=-1, **kw):
    return lib.ss_scan_fwd_states(ctypes.byref(scan_args(**kw)), states, time_step, None)


def test_scan_states_validation(lib):
    assert states_call(lib, states=None) == NULL
    assert states_call(lib, time_step=64) == SHAPE          # past the last token
    assert states_call(lib, time_step=1 << 40) == SHAPE
    assert states_call(lib, states=8 * MB + 2) == ALIGN
    assert states_call(lib, states=6 * MB) == ALIAS          # over y
    assert states_call(lib, states=1 * MB + 64) == ALIAS     # over x
    assert states_call(lib, h_last=9 * MB, states=9 * MB) == ALIAS
    # the checked span is every state (batch*channels*L*N floats) or one step's (batch*channels*N)
    every, one = 2 * 8 * 64 * 16 * 4, 2 * 8 * 16 * 4
    assert states_call(lib, states=6 * MB - every + 4) == ALIAS               # its last float is y's first
    assert states_call(lib, states=6 * MB - one + 4, time_step=5) == ALIAS
    assert states_call(lib, states=6 * MB - every + 4, time_step=5, batch=1 << 40, channels=1 << 40) == SHAPE
    assert states_call(lib, io=3) == DTYPE
    assert states_call(lib, batch=0) == OK                   # an empty problem is a no-op


def gated_call(lib, batch=2, L=64, dk=32, dv=16, io=1, sdt=0, q=1 * MB, k=2 * MB, v=3 * MB, gamma=4 * MB, s0=None,
               y=5 * MB, final_state=None):
    return lib.ss_gated_scan(batch, L, dk, dv, io, sdt, q, k, v, gamma, s0, y, final_state, None)


def test_gated_validation(lib):
    assert gated_call(lib, io=5) == DTYPE
    assert gated_call(lib, sdt=2) == DTYPE
    assert gated_call(lib, s0=6 * MB + 2) == ALIGN                       # fp32 state
    assert gated_call(lib, sdt=1, s0=6 * MB + 1) == ALIGN                 # bf16 state
    assert gated_call(lib, L=-1) == SHAPE
    assert gated_call(lib, dk=0) == UNSUP
    assert gated_call(lib, dk=257) == UNSUP
    assert gated_call(lib, dv=0) == UNSUP
    assert gated_call(lib, q=None) == NULL
    assert gated_call(lib, gamma=None) == NULL
    assert gated_call(lib, q=1 * MB + 1) == ALIGN
    assert gated_call(lib, gamma=4 * MB + 2) == ALIGN
    assert gated_call(lib, y=1 * MB) == ALIAS                              # y over q
    assert gated_call(lib, final_state=3 * MB + 4) == ALIAS                # final_state over v
    assert gated_call(lib, s0=6 * MB, final_state=6 * MB + 4) == ALIAS     # partial overlap with s0
    assert gated_call(lib, batch=1 << 40, L=1 << 40) == SHAPE
    assert gated_call(lib, batch=0) == OK


def attn_call(lib, batch=2, channels=3, N=16, L=64, io=1, dt=1 * MB, A=2 * MB, B=3 * MB, C=4 * MB,
              dt_bias=None, per_state=0, M=6 * MB):
    return lib.ss_effective_attention(batch, channels, N, L, io, dt, A, B, C, dt_bias, 1, 0, per_state, M, None)


def test_attention_validation(lib):
    assert attn_call(lib, io=7) == DTYPE
    assert attn_call(lib, L=-1) == SHAPE
    assert attn_call(lib, N=0) == UNSUP
    assert attn_call(lib, N=65) == UNSUP
    assert attn_call(lib, dt=None) == NULL
    assert attn_call(lib, M=None) == NULL
    assert attn_call(lib, B=3 * MB + 1) == ALIGN
    assert attn_call(lib, M=6 * MB + 2) == ALIGN
    assert attn_call(lib, M=1 * MB) == ALIAS                     # M over dt
    assert attn_call(lib, M=4 * MB - 16) == ALIAS                # M runs into C
    assert attn_call(lib, L=1 << 31, channels=1 << 20) == SHAPE  # M's bytes overflow
    assert attn_call(lib, batch=0) == OK
    assert attn_call(lib, L=0) == OK


def conv_call(lib, batch=2, channels=3, L=64, W=4, io=1, x_pre=1 * MB, w=2 * MB, b=None, reset=None, x=4 * MB):
    return lib.ss_conv1d_silu(batch, channels, L, W, io, x_pre, w, b, reset, x, None)


def proj_call(lib, batch=2, channels=64, L=64, R=16, io=1, w=1 * MB, delta=2 * MB, bias=None, dt=4 * MB):
    return lib.ss_dt_proj(batch, channels, L, R, io, w, delta, bias, 1, dt, None)


def test_producer_validation(lib):
    assert conv_call(lib, io=9) == DTYPE
    assert conv_call(lib, W=0) == UNSUP
    assert conv_call(lib, W=9) == UNSUP
    assert conv_call(lib, L=-1) == SHAPE
    assert conv_call(lib, x_pre=None) == NULL
    assert conv_call(lib, w=None) == NULL
    assert conv_call(lib, x=4 * MB + 1) == ALIGN
    assert conv_call(lib, w=2 * MB + 2) == ALIGN
    assert conv_call(lib, x=1 * MB + 2) == ALIAS        # x over x_pre
    assert conv_call(lib, reset=4 * MB + 100) == ALIAS  # reset inside x
    assert conv_call(lib, batch=0) == OK
    assert proj_call(lib, io=9) == DTYPE
    assert proj_call(lib, R=0) == UNSUP
    assert proj_call(lib, delta=None) == NULL
    assert proj_call(lib, dt=4 * MB + 1) == ALIGN
    assert proj_call(lib, bias=3 * MB + 2) == ALIGN
    assert proj_call(lib, dt=2 * MB) == ALIAS           # dt over delta
    assert proj_call(lib, L=0) == OK


def test_update_validation(lib):
    assert upd_call(lib, io=7) == DTYPE
    assert upd_call(lib, N=65) == UNSUP
    assert upd_call(lib, state=None) == NULL
    assert upd_call(lib, y=2 * MB) == ALIAS
    assert upd_call(lib, state=2 * MB) == ALIAS
    assert upd_call(lib, state=1 * MB + 2) == ALIGN
    assert upd_call(lib, batch=0) == OK


def test_binding_requires_device_tensors():
    import torch
    x = torch.zeros(1, 2, 3)
    with pytest.raises(ValueError):
        ss.ss_scan_fwd(x, x, torch.zeros(2, 4), torch.zeros(1, 4, 3), torch.zeros(1, 4, 3))


def test_validator_header_builds_standalone(tmp_path):
    """The validation header has no HIP dependency (host-only g++ build)."""
    src = tmp_path / "t.cpp"
    src.write_text('#include "ss_validate.h"\nint main(){ss_scan_args a{}; bool n; return ss::validate_scan(a,&n)==SS_ERR_UNSUPPORTED?0:1;}\n')
    exe = tmp_path / "t"
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-I",
                    os.path.join(ROOT, "selective_state_space_ss_amd", "csrc"), str(src), "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0


def _device_visible() -> bool:
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_launch_without_a_device_returns_hip_error(lib):
    """With no GPU present, valid calls get past validation and the failed
    launch comes back as SS_ERR_HIP rather than a crash. The pointers here are
    fake, so the test never runs where a GPU is visible."""
    if _device_visible():
        pytest.skip("a GPU is visible: this test launches with fake pointers")
    assert scan_call(lib) == HIP
    assert scan_call(lib, io=0, z=7 * MB, h0=8 * MB, h_last=9 * MB, reset=10 * MB) == HIP
    assert states_call(lib) == HIP
    assert states_call(lib, time_step=3) == HIP
    assert conv_scan_call(lib) == HIP
    assert conv_scan_call(lib, reset=10 * MB, width=7) == HIP
    assert upd_call(lib) == HIP
    assert gated_call(lib) == HIP
    assert attn_call(lib) == HIP
    assert conv_call(lib) == HIP
    assert proj_call(lib) == HIP
