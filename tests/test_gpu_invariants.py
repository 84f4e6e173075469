"""GPU invariants that hold at any size: decode steps against the scan,
split scans with the carried state, packed rows against per-document scans,
run-to-run determinism, untouched inputs, h_last written over h0, and the
error paths of the C ABI."""
import pytest
import torch

import selective_state_space_ss_amd as ss
from selective_state_space_ss_amd.workloads import make_case
from tests.helpers import SCAN_KERNELS, TOL, TOL_STATE, check_close, force_scan_kernel, np64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(params=SCAN_KERNELS)
def scan_kernel(request, monkeypatch):
    """Every prompt-scan kernel variant (tests/helpers.py, SCAN_KERNELS)."""
    force_scan_kernel(monkeypatch, request.param)
    return request.param


def scan(d, **kw):
    args = dict(D=d["D"], z=d.get("z"), dt_bias=d["dt_bias"], h0=d.get("h0"), reset=d.get("reset"))
    args.update(kw)
    return ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], **args)


def test_decode_steps_equal_scan(scan_kernel):
    """nnterp "selective_scan" page: the decode call continues from the cached
    state; T decode steps reproduce a T-token scan."""
    d = to_dev(make_case(501, 2, 21, 16, 40, "f32", gate=True, h0=True))
    y, h = scan(d)
    state = d["h0"].clone()
    ys = []
    for t in range(d["x"].shape[2]):
        ys.append(ss.ss_state_update(state, d["x"][:, :, t].contiguous(), d["dt"][:, :, t].contiguous(), d["A"],
                                     d["B"][:, :, t].contiguous(), d["C"][:, :, t].contiguous(), D=d["D"],
                                     z=d["z"][:, :, t].contiguous(), dt_bias=d["dt_bias"]))
    torch.cuda.synchronize()
    check_close(np64(torch.stack(ys, dim=2)), np64(y), *TOL["f32"], "decode x T vs scan")
    check_close(np64(state), np64(h), *TOL_STATE, "decode state vs h_last")


@pytest.mark.parametrize("L1", [0, 1, 255, 256, 700, 1023])
def test_split_scan_with_carried_state(L1, scan_kernel):
    d = to_dev(make_case(502, 2, 18, 16, 1500, "bf16", gate=True, h0=True, reset_mean_doc=300))
    y, h = scan(d)
    part = lambda t, s, e: None if t is None else t[..., s:e].contiguous()
    L = d["x"].shape[2]
    y1, h1 = ss.ss_scan_fwd(part(d["x"], 0, L1), part(d["dt"], 0, L1), d["A"], part(d["B"], 0, L1),
                            part(d["C"], 0, L1), D=d["D"], z=part(d["z"], 0, L1), dt_bias=d["dt_bias"], h0=d["h0"],
                            reset=part(d["reset"], 0, L1))
    y2, h2 = ss.ss_scan_fwd(part(d["x"], L1, L), part(d["dt"], L1, L), d["A"], part(d["B"], L1, L),
                            part(d["C"], L1, L), D=d["D"], z=part(d["z"], L1, L), dt_bias=d["dt_bias"], h0=h1,
                            reset=part(d["reset"], L1, L))
    torch.cuda.synchronize()
    check_close(np64(torch.cat([y1, y2], dim=2)), np64(y), *TOL["bf16"], f"split at {L1}")
    check_close(np64(h2), np64(h), *TOL_STATE, f"split state at {L1}")


def test_packed_row_equals_document_scans(scan_kernel):
    """"s6_reset" post, Sequence Packing: with hard resets a packed row equals
    zero-state scans of its documents."""
    d = to_dev(make_case(503, 1, 20, 16, 1100, "f32", gate=True, h0=True))
    starts = [0, 1, 333, 334, 700, 1099]
    reset = torch.zeros(1, 1100, dtype=torch.uint8, device="cuda")
    reset[0, starts] = 1
    y, h = scan(d, reset=reset)
    bounds = starts + [1100]
    for s, e in zip(bounds[:-1], bounds[1:]):
        part = lambda t: t[..., s:e].contiguous()
        yd, hd = ss.ss_scan_fwd(part(d["x"]), part(d["dt"]), d["A"], part(d["B"]), part(d["C"]), D=d["D"],
                                z=part(d["z"]), dt_bias=d["dt_bias"])
        torch.cuda.synchronize()
        check_close(np64(yd), np64(y[..., s:e]), *TOL["f32"], f"document {s}:{e}")
    check_close(np64(hd), np64(h), *TOL_STATE, "last document state")


def test_deterministic_and_inputs_untouched(scan_kernel):
    d = to_dev(make_case(504, 3, 40, 16, 2048, "bf16", gate=True, h0=True, reset_mean_doc=200))
    before = {k: v.clone() for k, v in d.items() if v is not None}
    y1, h1 = scan(d)
    y2, h2 = scan(d)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    for k, v in before.items():
        assert torch.equal(v, d[k]), f"input {k} was modified"


def test_h_last_may_overwrite_h0(scan_kernel):
    d = to_dev(make_case(505, 2, 33, 16, 700, "bf16", gate=True, h0=True))
    y_ref, h_ref = scan(d)
    h = d["h0"].clone()
    y, h_out = scan(d, h0=h, h_last=h)
    torch.cuda.synchronize()
    assert h_out.data_ptr() == h.data_ptr()
    assert torch.equal(y, y_ref) and torch.equal(h, h_ref)


def test_c_abi_errors():
    d = to_dev(make_case(506, 1, 4, 16, 64, "bf16"))
    with pytest.raises(ss.SSError) as e:  # y overlapping x
        scan(d, y=d["x"])
    assert e.value.code == 5
    bad_A = torch.zeros(4, 65, device="cuda")
    B65 = torch.zeros(1, 65, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ss.SSError) as e:
        ss.ss_scan_fwd(d["x"], d["dt"], bad_A, B65, B65)
    assert e.value.code == 4
    with pytest.raises(ValueError):
        ss.ss_scan_fwd(d["x"].cpu(), d["dt"], d["A"], d["B"], d["C"])
