"""The learned-like A of the GPU parity cases in test_gpu_general_A.py tells
channels apart, which the S4D-real A cannot: a kernel that read A of the
wrong channel (here planted in the oracle's inputs, channel c reading channel
0's row) is far outside the parity bar on the learned A and invisible on
the S4D-real one (every channel's row is the same)."""
import numpy as np

from selective_state_space_ss_amd.workloads import make_case
from tests.helpers import TOL, np64, oracle_scan_full


def _outside_bar(inp):
    ref_y, ref_h = oracle_scan_full(inp)
    wrong = dict(inp)
    wrong["A"] = inp["A"][:1].expand_as(inp["A"]).contiguous()
    y, h = oracle_scan_full(wrong)
    rtol, atol = TOL["bf16"]
    return float((np.abs(y - ref_y) / (atol + rtol * np.abs(ref_y))).max())


def test_learned_A_detects_a_wrong_channel():
    inp = make_case(4117, 2, 40, 16, 1777, "bf16", gate=True, h0=True, dt_bias="loguniform", a_init="learned")
    assert not np.allclose(np64(inp["A"][0]), np64(inp["A"][1]))
    assert _outside_bar(inp) > 10.0


def test_s4d_real_A_cannot():
    inp = make_case(4117, 2, 40, 16, 1777, "bf16", gate=True, h0=True, dt_bias="loguniform")
    assert _outside_bar(inp) == 0.0


def test_learned_A_recipe():
    A = np64(make_case(4117, 1, 40, 16, 8, "f32", a_init="learned")["A"])
    assert A.shape == (40, 16) and (A <= 0).all()
    assert (A == 0).any() and (A == -5000.0).any()
    mid = A[(A < 0) & (A > -5000.0)]
    assert 0.5 < np.median(-mid) < 4.0 and (-mid).max() > 20.0
