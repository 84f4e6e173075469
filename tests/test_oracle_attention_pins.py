"""Pins of the oracle's effective attention (TransformerLens "ssm_mixer" page,
compute_effective_attention:
M[c, i, j] = sum_n C[i, n] prod_{k=j+1..i} exp(A[c, n] dt[c, k]) B[j, n], causal)
against routes of their own: the selective scan itself (the page's
reconstruction y = M x + D x, pre-gate, with dt scaling), the product
written as the exponential of a sum, the decay-free special case as a plain
matrix product, the unsummed form, and a hand-worked case."""
import math

import numpy as np
import pytest

import oracle


def rand_case(seed, batch=2, channels=3, N=4, L=13, softplus=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((batch, channels, L)),
                dt=rng.standard_normal((batch, channels, L)),
                A=-rng.uniform(0.2, 3.0, (channels, N)),
                B=rng.standard_normal((batch, N, L)),
                C=rng.standard_normal((batch, N, L)),
                D=rng.standard_normal(channels),
                dt_bias=rng.uniform(-1.0, 0.5, channels),
                softplus=softplus)


def step_sizes(c):
    v = c["dt"] + c["dt_bias"][None, :, None]
    return np.logaddexp(0.0, v) if c["softplus"] else v


def attn(c, **kw):
    return oracle.effective_attention(c["dt"], c["A"], c["B"], c["C"], dt_bias=c["dt_bias"],
                                      dt_softplus=c["softplus"], **kw)


def close(a, b, rtol=1e-12, atol=1e-12):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


@pytest.mark.parametrize("softplus", [True, False])
def test_apin1_reconstructs_the_scan(softplus):
    """ssm_mixer page, include_dt_scaling: y[c, i] = sum_j M[c, i, j] x[c, j]
    + D[c] x[c, i] is the scan's output before the gate, here the oracle's
    own token loop (zero initial state, no gate)."""
    c = rand_case(11, softplus=softplus)
    y, _ = oracle.scan(c["x"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], dt_bias=c["dt_bias"],
                       dt_softplus=softplus)
    M = attn(c, include_dt_scaling=True)
    y_ref = np.einsum("bcij,bcj->bci", M, c["x"]) + c["D"][None, :, None] * c["x"]
    close(y, y_ref, rtol=1e-11, atol=1e-11)


def test_apin2_product_as_exponential_of_a_sum():
    """prod_{k=j+1..i} exp(A dt_k) = exp(A * (sum_{k<=i} dt_k - sum_{k<=j} dt_k)),
    with numpy's cumsum; zero above the diagonal."""
    c = rand_case(12, batch=1, channels=2, N=3, L=10)
    d = step_sizes(c)[0]                                 # [c, L]
    cs = np.cumsum(d, axis=1)
    L = d.shape[1]
    diff = cs[:, :, None] - cs[:, None, :]               # [c, i, j]
    causal = np.tril(np.ones((L, L), dtype=bool))
    decay = np.exp(c["A"][:, :, None, None] * diff[:, None]) * causal   # [c, n, i, j]
    M_ref = np.einsum("ni,cnij,nj->cij", c["C"][0], decay, c["B"][0])
    close(attn(c)[0], M_ref, rtol=1e-11, atol=1e-12)


def test_apin3_no_decay_is_a_masked_matrix_product():
    """A = 0: every decay factor is 1, so M = tril(C^T B) (numpy matmul),
    and with dt scaling each column j times dt_j."""
    c = rand_case(13, batch=2, channels=2, N=5, L=9)
    c["A"][:] = 0.0
    d = step_sizes(c)
    M = attn(c)
    Md = attn(c, include_dt_scaling=True)
    for b in range(2):
        P = np.tril(c["C"][b].T @ c["B"][b])
        for ch in range(2):
            close(M[b, ch], P)
            close(Md[b, ch], P * d[b, ch][None, :])


def test_apin4_causal_zeros_and_diagonal():
    """Above the diagonal M is exactly 0; on it the product is empty, so
    M[i, i] = sum_n C[i, n] B[i, n]."""
    c = rand_case(14, L=15)
    M = attn(c)
    L = 15
    upper = np.triu(np.ones((L, L), dtype=bool), 1)
    assert np.all(M[:, :, upper] == 0.0)
    diag = np.einsum("bni,bni->bi", c["C"], c["B"])
    for ch in range(3):
        close(np.diagonal(M[:, ch], axis1=1, axis2=2), diag, rtol=1e-14, atol=1e-14)


def test_apin5_unsummed_form():
    """per_state_coord: the [.., N, L, L] terms sum over n to M; term n alone is
    the N = 1 attention of coordinate n (its own A column, B and C rows)."""
    c = rand_case(15, N=3, L=11)
    Mn = attn(c, per_state_coord=True)
    assert Mn.shape == (2, 3, 3, 11, 11)
    close(Mn.sum(axis=2), attn(c))
    for n in range(3):
        cn = dict(c, A=c["A"][:, n:n + 1], B=c["B"][:, n:n + 1], C=c["C"][:, n:n + 1])
        close(Mn[:, :, n], attn(cn)[:, :, :, :])


def test_apin6_hand_worked_case():
    """One channel, one state coordinate, step size 1 without softplus, A =
    -ln 2 (decay 1/2 per token), B = (1, 2, 4), C = (1, 1, 3):
        M = [[1*1, 0, 0], [1*(1/2)*1, 1*2, 0], [3*(1/4)*1, 3*(1/2)*2, 3*4]]
          = [[1, 0, 0], [0.5, 2, 0], [0.75, 3, 12]]."""
    c = dict(dt=np.ones((1, 1, 3)), A=np.array([[-math.log(2.0)]]), B=np.array([[[1.0, 2.0, 4.0]]]),
             C=np.array([[[1.0, 1.0, 3.0]]]), dt_bias=np.zeros(1), softplus=False)
    M = attn(c)[0, 0]
    close(M, np.array([[1.0, 0.0, 0.0], [0.5, 2.0, 0.0], [0.75, 3.0, 12.0]]), rtol=1e-15, atol=1e-15)


def test_apin7_channel_and_batch_permutation():
    """Rows are independent: permuting channels (with A, dt_bias) or batch
    items (with B, C) permutes M the same way."""
    c = rand_case(16, batch=3, channels=4)
    M = attn(c)
    pc = np.array([2, 0, 3, 1])
    cc = dict(c, dt=c["dt"][:, pc], A=c["A"][pc], dt_bias=c["dt_bias"][pc])
    close(attn(cc), M[:, pc], rtol=0, atol=0)
    pb = np.array([1, 2, 0])
    cb = dict(c, dt=c["dt"][pb], B=c["B"][pb], C=c["C"][pb])
    close(attn(cb), M[pb], rtol=0, atol=0)
