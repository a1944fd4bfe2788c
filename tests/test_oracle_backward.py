"""Pins for the attention-gradient oracle (oracle/backward.py).

The gradients are checked against central finite differences of the forward
oracle (an independent evaluation: only oracle.head's forward values enter), on
tiny shapes, causal and not, N_q != N_kv; plus closed forms and planted mistakes.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as obwd

RNG = np.random.default_rng(4242)


def loss(q, k, v, w, scale, causal):
    o, _ = oracle.head(q, k, v, scale, causal)
    return float((o * w).sum())


def finite_diff(q, k, v, w, scale, causal, h=1e-6):
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            up = loss(q, k, v, w, scale, causal)
            x[idx] = old - h
            dn = loss(q, k, v, w, scale, causal)
            x[idx] = old
            g[idx] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nkv", [(3, 3), (4, 6), (5, 2), (1, 7)])
def test_gradients_match_finite_differences(causal, nq, nkv):
    d = 4
    q, k, v, w = (RNG.standard_normal(s) for s in ((nq, d), (nkv, d), (nkv, d), (nq, d)))
    dq, dk, dv, _ = obwd.head_backward(q, k, v, w, 0.8, causal)
    fq, fk, fv = finite_diff(q, k, v, w, 0.8, causal)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-7)


def test_delta_is_rowsum_of_do_times_o():
    q, k, v, w = (RNG.standard_normal(s) for s in ((5, 8), (9, 8), (9, 8), (5, 8)))
    _, _, _, dd = obwd.head_backward(q, k, v, w, 0.5, True)
    o, _ = oracle.head(q, k, v, 0.5, True)
    np.testing.assert_allclose(dd, (w * o).sum(axis=1), rtol=0, atol=1e-13)


def test_closed_forms():
    """One key: O = v_0 for every query, so dV_0 = sum_i dO_i and dQ = dK = 0."""
    q, k, v, w = (RNG.standard_normal(s) for s in ((6, 4), (1, 4), (1, 4), (6, 4)))
    dq, dk, dv, _ = obwd.head_backward(q, k, v, w, 1.3, False)
    np.testing.assert_allclose(dv[0], w.sum(axis=0), rtol=0, atol=1e-13)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    # Softmax weights sum to one, so shifting every key by the same vector c changes
    # the scores of row i by the same q_i . c: the gradient of K summed over keys is 0.
    q, k, v, w = (RNG.standard_normal(s) for s in ((5, 4), (7, 4), (7, 4), (5, 4)))
    _, dk, _, _ = obwd.head_backward(q, k, v, w, 0.7, False)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # Rows with no visible key (causal, N_q > N_kv) contribute nothing.
    q, k, v, w = (RNG.standard_normal(s) for s in ((6, 4), (2, 4), (2, 4), (6, 4)))
    dq, dk, dv, _ = obwd.head_backward(q, k, v, w, 0.7, True)
    assert np.all(dq[:4] == 0)
    w2 = w.copy()
    w2[:4] = 100.0
    _, dk2, dv2, _ = obwd.head_backward(q, k, v, w2, 0.7, True)
    np.testing.assert_allclose(dk2, dk, atol=1e-13)
    np.testing.assert_allclose(dv2, dv, atol=1e-13)


def _mutant(kind):
    def f(q, k, v, w, scale, causal):
        s = scale * (q @ k.T)
        if causal:
            j = np.arange(k.shape[0])[None, :]
            s = np.where(j > np.arange(q.shape[0])[:, None] + (k.shape[0] - q.shape[0]), -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v
        dp = w @ v.T
        d = (w * o).sum(axis=1)
        ds = p * (dp - d[:, None]) if kind != "no_delta" else p * dp
        dq = scale * (ds @ k) if kind != "no_scale" else ds @ k
        dk = scale * (ds.T @ q) if kind != "transposed" else scale * (ds @ q[: k.shape[0]])
        dv = p.T @ w
        return dq, dk, dv
    return f


@pytest.mark.parametrize("kind", ["no_delta", "no_scale", "transposed"])
def test_finite_differences_catch_planted_mistakes(kind):
    q, k, v, w = (RNG.standard_normal(s) for s in ((4, 4), (4, 4), (4, 4), (4, 4)))
    got = _mutant(kind)(q, k, v, w, 0.9, False)
    ref = finite_diff(q, k, v, w, 0.9, False)
    assert any(np.abs(a - b).max() > 1e-5 for a, b in zip(got, ref))


def test_batched_matches_heads():
    q, k, v, w = (RNG.standard_normal(s) for s in ((2, 3, 5, 4), (2, 3, 7, 4), (2, 3, 7, 4), (2, 3, 5, 4)))
    dq, dk, dv, dd = oracle.attention_backward(q, k, v, w, 0.6, True)
    h = obwd.head_backward(q[1, 2], k[1, 2], v[1, 2], w[1, 2], 0.6, True)
    for a, b in zip((dq[1, 2], dk[1, 2], dv[1, 2], dd[1, 2]), h):
        np.testing.assert_array_equal(a, b)
