"""GPU parity of ss_scan_fwd_states: the state after every token (nnterp
"selective_scan" page, the `states` attribute; here [batch, channels,
state_dim, seq], the oracle's [.., seq, state_dim] transposed) and after one
selected token
(TransformerLens "ssm_mixer" page, compute_ssm_state(time_step)) against the
fp64 oracle's per-token states; y and h_last are bitwise those of
ss_scan_fwd in its plain chunked form (the same kernel with the state
output switched off; the forms for few rows, which ss_scan_fwd picks at
these small shapes, combine in another order, so the module forces the plain
form through SS_SCAN_FORM=plain).

The states are fp32 for every I/O type and are held to the fp32 bar."""
import pytest
import torch

import oracle
import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import make_case
from tests.helpers import TOL_STATE, check_close, np64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def plain_scan_form(monkeypatch):
    monkeypatch.setenv("SS_SCAN_FORM", "plain")


def oracle_states(inp):
    return oracle.scan(np64(inp["x"]), np64(inp["dt"]), np64(inp["A"]), np64(inp["B"]), np64(inp["C"]),
                       D=np64(inp["D"]), z=np64(inp.get("z")), dt_bias=np64(inp["dt_bias"]),
                       h0=np64(inp.get("h0")), reset=None if inp.get("reset") is None else inp["reset"].numpy(),
                       return_states=True)


def run(d, **kw):
    return ss.ss_scan_fwd_states(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d.get("z"),
                                 dt_bias=d["dt_bias"], h0=d.get("h0"), reset=d.get("reset"), **kw)


CASES = [
    # io, batch, channels, N, L, gate, h0, reset mean
    ("f32", 2, 19, 16, 300, True, True, 40),
    ("bf16", 2, 33, 16, 513, True, True, None),
    ("bf16", 1, 40, 4, 1030, False, False, 100),
    ("f32", 2, 7, 9, 257, True, True, None),
    ("bf16", 2, 17, 33, 600, True, True, 150),
    ("bf16", 1, 9, 64, 280, True, False, None),
]


@pytest.mark.parametrize("io,batch,channels,N,L,gate,h0,reset", CASES,
                         ids=[f"{c[0]}-b{c[1]}-c{c[2]}-N{c[3]}-L{c[4]}" for c in CASES])
def test_every_state(io, batch, channels, N, L, gate, h0, reset):
    print(f"states all io={io} b={batch} c={channels} N={N} L={L}", flush=True)
    inp = make_case(700 + L + N, batch, channels, N, L, io, gate=gate, h0=h0, reset_mean_doc=reset)
    d = to_dev(inp)
    y, h, st = run(d)
    y0, h0_ = ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d.get("z"), dt_bias=d["dt_bias"],
                             h0=d.get("h0"), reset=d.get("reset"))
    torch.cuda.synchronize()
    yr, hr, sr = oracle_states(inp)
    assert st.shape == (batch, channels, N, L)
    check_close(np64(st), sr.transpose(0, 1, 3, 2), *TOL_STATE, f"states {io} N={N} L={L}")
    check_close(np64(h), hr, *TOL_STATE, "h_last")
    assert torch.equal(y, y0) and torch.equal(h, h0_), "y / h_last differ from ss_scan_fwd"
    # the walk's last state and the carried h_last round differently (the
    # carry comes out of the lane scan), so they agree to the fp32 bar only
    check_close(np64(st[..., -1]), np64(h), *TOL_STATE, "last state vs h_last")


@pytest.mark.parametrize("t", [0, 1, 15, 16, 255, 256, 511, 700, 1029])
def test_one_state(t):
    """The selected token at chunk and lane boundaries and the last token."""
    print(f"states one t={t}", flush=True)
    inp = make_case(790, 2, 21, 16, 1030, "bf16", gate=True, h0=True, reset_mean_doc=120)
    d = to_dev(inp)
    y, h, st = run(d, time_step=t)
    y0, _ = ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], dt_bias=d["dt_bias"],
                           h0=d["h0"], reset=d["reset"])
    torch.cuda.synchronize()
    _, _, sr = oracle_states(inp)
    assert st.shape == (2, 21, 16)
    check_close(np64(st), sr[:, :, t], *TOL_STATE, f"state after token {t}")
    assert torch.equal(y, y0)


def test_one_state_wide_and_unaligned_length():
    """state_dim 40 (the 64-wide instance: four groups of 16, the last ones past N) and a
    length that is not a multiple of the vector width."""
    inp = make_case(791, 1, 12, 40, 333, "f32", gate=False, h0=True, reset_mean_doc=None)
    d = to_dev(inp)
    _, _, sr = oracle_states(inp)
    for t in (0, 200, 332):
        _, _, st = run(d, time_step=t)
        torch.cuda.synchronize()
        check_close(np64(st), sr[:, :, t], *TOL_STATE, f"N=40 state after token {t}")


def test_states_errors():
    inp = make_case(792, 1, 4, 16, 64, "bf16")
    d = to_dev(inp)
    with pytest.raises(ss.SSError) as e:
        run(d, time_step=64)
    assert e.value.code == 2
    with pytest.raises(ValueError):
        run(d, time_step=-3)
    states = torch.empty(1, 4, 16, 64, device="cuda")
    y_over_states = states.view(-1).view(torch.bfloat16)[:256].view(1, 4, 64)
    with pytest.raises(ss.SSError) as e:
        run(d, y=y_over_states, states=states)
    assert e.value.code == 5
