"""Race check of the chunked scan's LDS stage (the debug library
libssscan_lds_poison.so, built with SS_LDS_POISON=1): before every fill of
the B/C stage the kernel writes NaN over the whole stage between two
barriers, so a read not ordered after the fill, or a fill racing a previous
chunk's reader, shows up as NaN or as a changed value. Every launch form of
the chunked kernel (plain, the 32- and 64-lane rows, 16 and 32 tokens per
lane with resets, more than one coordinate group, the every-token states and
the fused conv) must give outputs bitwise equal to the normal library's."""
import ctypes

import pytest
import torch

import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd import _binding as bd
from selective_state_space_ss_amd.build import POISON_LIB
from selective_state_space_ss_amd.workloads import make_case, make_producer_case
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

_poison = None


def poison_lib():
    global _poison
    if _poison is None:
        lib = ctypes.CDLL(POISON_LIB)
        lib.ss_scan_fwd.restype = ctypes.c_int
        lib.ss_scan_fwd.argtypes = [ctypes.POINTER(bd.ScanArgs), ctypes.c_void_p]
        lib.ss_scan_fwd_states.restype = ctypes.c_int
        lib.ss_scan_fwd_states.argtypes = [ctypes.POINTER(bd.ScanArgs), ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_void_p]
        lib.ss_scan_fwd_conv.restype = ctypes.c_int
        lib.ss_scan_fwd_conv.argtypes = [ctypes.POINTER(bd.ScanArgs), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p]
        _poison = lib
    return _poison


def stream():
    return torch.cuda.current_stream().cuda_stream


def poison_scan(d):
    y, h, args, _ = bd._scan_args(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d.get("z"), d["dt_bias"],
                                  d.get("h0"), d.get("reset"), True, None, None, True)
    assert poison_lib().ss_scan_fwd(ctypes.byref(args), stream()) == bd.SS_OK
    return y, h


def normal_scan(d):
    return ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d.get("z"), dt_bias=d["dt_bias"],
                          h0=d.get("h0"), reset=d.get("reset"))


def assert_same(got, ref, what):
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert not torch.isnan(g.float()).any(), f"{what}: NaN from the poisoned stage"
        assert torch.equal(g, r), f"{what}: differs from the normal build"


CASES = [
    # (label, env, batch, channels, state_dim, seq, io, reset mean doc)
    ("plain bf16", {"SS_SCAN_FORM": "plain"}, 2, 70, 16, 1100, "bf16", None),
    ("plain fp32, 4 groups of 16", {"SS_SCAN_FORM": "plain"}, 1, 36, 40, 700, "f32", None),
    ("rows of 32 lanes, 4 waves", {"SS_SCAN_FORM": "r32w4"}, 2, 50, 16, 1300, "bf16", None),
    ("rows of 32 lanes, 8 waves", {"SS_SCAN_FORM": "r32w8"}, 2, 40, 9, 900, "bf16", None),
    ("rows of 64 lanes", {"SS_SCAN_FORM": "r64w4"}, 1, 30, 16, 2300, "bf16", None),
    ("resets, K = 16", {"SS_SCAN_TOKENS_PER_LANE": "16"}, 2, 40, 16, 1200, "bf16", 200),
    ("resets, K = 32", {"SS_SCAN_TOKENS_PER_LANE": "32"}, 2, 40, 16, 1500, "bf16", 200),
]


@pytest.mark.parametrize("label,env,batch,channels,n,L,io,doc", CASES, ids=[c[0] for c in CASES])
def test_poisoned_stage_scan(label, env, batch, channels, n, L, io, doc, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    d = to_dev(make_case(880 + len(label), batch, channels, n, L, io, gate=True, h0=True, reset_mean_doc=doc))
    assert_same(poison_scan(d), normal_scan(d), label)


def test_poisoned_stage_states():
    d = to_dev(make_case(891, 2, 40, 16, 600, "bf16", gate=True, h0=True, reset_mean_doc=150))
    ref = ss.ss_scan_fwd_states(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], dt_bias=d["dt_bias"],
                                h0=d["h0"], reset=d["reset"])
    y, h, args, _ = bd._scan_args(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"], d["h0"],
                                  d["reset"], True, None, None, True)
    st = torch.empty_like(ref[2])
    assert poison_lib().ss_scan_fwd_states(ctypes.byref(args), ctypes.c_void_p(st.data_ptr()), -1,
                                           stream()) == bd.SS_OK
    assert_same((y, h, st), ref, "every-token states")


def test_poisoned_stage_fused_conv():
    batch, channels, L, W = 2, 48, 900, 4
    pc = make_producer_case(892, batch, channels, L, W, 16, "bf16", device="cuda")
    d = to_dev(make_case(893, batch, channels, 16, L, "bf16", gate=True, h0=True, reset_mean_doc=200))
    ref = ss.ss_scan_fwd_conv(pc["x_pre"], d["dt"], d["A"], d["B"], d["C"], pc["conv_w"], pc["conv_b"], D=d["D"],
                              z=d["z"], dt_bias=d["dt_bias"], h0=d["h0"], reset=d["reset"])
    y, h, args, _ = bd._scan_args(pc["x_pre"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"],
                                  d["h0"], d["reset"], True, None, None, True)
    assert poison_lib().ss_scan_fwd_conv(ctypes.byref(args), ctypes.c_void_p(pc["conv_w"].data_ptr()),
                                         ctypes.c_void_p(pc["conv_b"].data_ptr()), W, stream()) == bd.SS_OK
    assert_same((y, h), ref, "fused conv")
