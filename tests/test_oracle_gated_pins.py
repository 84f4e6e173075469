"""Pins of the oracle's scalar-gated state scan ("Mamba 2 Gated State Scan"
problem page: S_t = gamma_t S_{t-1} + k_t v_t^T, y_t = q_t^T S_t, from a zero
state) against facts computed by routes of their own: the unrolled sum,
prefix sums, hand-worked cases, and the special case in which the selective
scan of the nnterp "selective_scan" page is the same recurrence (one decay
for every channel and state coordinate)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gated_hand_cases.json")


def rand_case(seed, batch=2, L=13, dk=3, dv=4, s0=True, zeros=False):
    rng = np.random.default_rng(seed)
    gamma = rng.uniform(0.0, 1.0, (batch, L))
    if zeros:
        gamma[rng.random((batch, L)) < 0.25] = 0.0
    return dict(q=rng.standard_normal((batch, L, dk)), k=rng.standard_normal((batch, L, dk)),
                v=rng.standard_normal((batch, L, dv)), gamma=gamma,
                s0=rng.standard_normal((batch, dk, dv)) if s0 else None)


def close(a, b, rtol=1e-12, atol=1e-12):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


@pytest.mark.parametrize("seed,zeros", [(1, False), (2, True), (3, True)])
def test_gpin1_unrolled_sum(seed, zeros):
    """S_t = prod_{i<=t} gamma_i S_0 + sum_{j<=t} prod_{i=j+1..t} gamma_i k_j v_j^T,
    each product written out, and y_t = q_t^T S_t."""
    c = rand_case(seed, zeros=zeros)
    y, fs = oracle.gated_scan(c["q"], c["k"], c["v"], c["gamma"], s0=c["s0"])
    batch, L, dk = c["q"].shape
    for b in range(batch):
        for t in range(L):
            S = np.prod(c["gamma"][b, :t + 1]) * c["s0"][b]
            for j in range(t + 1):
                S = S + np.prod(c["gamma"][b, j + 1:t + 1]) * np.outer(c["k"][b, j], c["v"][b, j])
            close(y[b, t], c["q"][b, t] @ S)
            if t == L - 1:
                close(fs[b], S)


def test_gpin2_reduces_to_the_selective_scan():
    """One decay a for every channel and state coordinate and one step size per
    token makes the selective scan (nnterp page, class docstring) this scan:
    h_t[c, n] = e^{dt_t a} h_{t-1}[c, n] + dt_t x_t[c] B_t[n] is S = h^T with
    gamma_t = e^{dt_t a}, k_t = B_t, v_t = dt_t x_t, and y_t[c] = C_t . h_t[c]
    is q_t^T S_t with q_t = C_t."""
    rng = np.random.default_rng(4)
    batch, channels, N, L, a = 2, 5, 3, 11, -0.7
    x = rng.standard_normal((batch, channels, L))
    d = rng.uniform(0.1, 1.5, (batch, L))
    Bm = rng.standard_normal((batch, N, L))
    Cm = rng.standard_normal((batch, N, L))
    h0 = rng.standard_normal((batch, channels, N))
    y1, h1 = oracle.scan(x, np.repeat(d[:, None, :], channels, axis=1), np.full((channels, N), a), Bm, Cm,
                         h0=h0, dt_softplus=False)
    y2, s2 = oracle.gated_scan(Cm.transpose(0, 2, 1), Bm.transpose(0, 2, 1), (d[:, None, :] * x).transpose(0, 2, 1),
                               np.exp(d * a), s0=h0.transpose(0, 2, 1))
    close(y2, y1.transpose(0, 2, 1), rtol=1e-11, atol=1e-11)
    close(s2, h1.transpose(0, 2, 1), rtol=1e-11, atol=1e-11)


def test_gpin3_unit_gate_is_a_prefix_sum():
    """gamma = 1: S_t = S_0 + cumsum of k_j v_j^T (numpy cumsum)."""
    c = rand_case(5)
    c["gamma"][:] = 1.0
    y, fs = oracle.gated_scan(c["q"], c["k"], c["v"], c["gamma"], s0=c["s0"])
    S = c["s0"][:, None] + np.cumsum(np.einsum("bti,btj->btij", c["k"], c["v"]), axis=1)
    close(y, np.einsum("bti,btij->btj", c["q"], S))
    close(fs, S[:, -1])


def test_gpin4_zero_gate_keeps_only_the_current_token():
    """gamma = 0: S_t = k_t v_t^T, so y_t = (q_t . k_t) v_t, whatever S_0."""
    c = rand_case(6)
    c["gamma"][:] = 0.0
    y, fs = oracle.gated_scan(c["q"], c["k"], c["v"], c["gamma"], s0=c["s0"])
    close(y, np.einsum("bti,bti->bt", c["q"], c["k"])[..., None] * c["v"])
    close(fs, np.einsum("bi,bj->bij", c["k"][:, -1], c["v"][:, -1]))


def _hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_gpin5_hand_worked_cases(case):
    """Hand-worked values (tests/golden/gated_hand_cases.json, each with its cite)."""
    arr = lambda k: None if k not in case else np.array(case[k], dtype=np.float64)
    y, fs = oracle.gated_scan(arr("q"), arr("k"), arr("v"), arr("gamma"), s0=arr("s0"))
    close(y, arr("expect_y"), rtol=0, atol=1e-15)
    close(fs, arr("expect_final_state"), rtol=0, atol=1e-15)


def test_gpin6_split_carries_the_state():
    """Running the first L1 tokens, then the rest from the state they leave,
    is the whole scan, bitwise (the same operations in the same order)."""
    c = rand_case(7, L=20, zeros=True)
    y, fs = oracle.gated_scan(c["q"], c["k"], c["v"], c["gamma"], s0=c["s0"])
    for L1 in (0, 1, 7, 19, 20):
        sl = lambda a, s, e: a[:, s:e]
        ya, sa = oracle.gated_scan(sl(c["q"], 0, L1), sl(c["k"], 0, L1), sl(c["v"], 0, L1),
                                   sl(c["gamma"], 0, L1), s0=c["s0"])
        yb, sb = oracle.gated_scan(sl(c["q"], L1, 20), sl(c["k"], L1, 20), sl(c["v"], L1, 20),
                                   sl(c["gamma"], L1, 20), s0=sa)
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y) and np.array_equal(sb, fs)


def test_gpin7_batch_items_are_independent():
    """Permuting the batch permutes the outputs (each item its own state)."""
    c = rand_case(8, batch=4)
    y, fs = oracle.gated_scan(c["q"], c["k"], c["v"], c["gamma"], s0=c["s0"])
    p = np.array([2, 0, 3, 1])
    yp, fsp = oracle.gated_scan(c["q"][p], c["k"][p], c["v"][p], c["gamma"][p], s0=c["s0"][p])
    assert np.array_equal(yp, y[p]) and np.array_equal(fsp, fs[p])


def test_gpin8_linear_in_values_and_initial_state():
    """For fixed q, k, gamma the outputs are linear in (v, S_0) jointly."""
    c = rand_case(9)
    c2 = rand_case(10)
    run = lambda v, s0: oracle.gated_scan(c["q"], c["k"], v, c["gamma"], s0=s0)
    ya, sa = run(c["v"], c["s0"])
    yb, sb = run(c2["v"], c2["s0"])
    yc, sc = run(2.0 * c["v"] - 3.0 * c2["v"], 2.0 * c["s0"] - 3.0 * c2["s0"])
    close(yc, 2.0 * ya - 3.0 * yb, rtol=1e-11, atol=1e-11)
    close(sc, 2.0 * sa - 3.0 * sb, rtol=1e-11, atol=1e-11)
