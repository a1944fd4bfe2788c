"""Pins for the float64 attention oracle.

Each check ties the oracle to something other than itself: a closed form, an
invariance the mathematics guarantees, or a brute-force evaluation at 50 digits
on tiny inputs. ``test_pins_catch_planted_mistakes`` plants plausible mistakes
in copies of the oracle and shows that at least one pin fails for each.
"""
import math

import mpmath
import numpy as np
import pytest

import oracle
from oracle import attention as oatt

RNG = np.random.default_rng(12345)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal):
    """Scalar mpmath evaluation of softmax(scale q k^T) v at 50 digits."""
    mpmath.mp.dps = 50
    nq, nkv = q.shape[0], k.shape[0]
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        vis = [j for j in range(nkv) if not causal or j <= i + (nkv - nq)]
        if not vis:
            lse[i] = -np.inf
            continue
        s = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i, t]) * mpmath.mpf(k[j, t])
                                                   for t in range(q.shape[1])) for j in vis}
        z = mpmath.fsum(mpmath.exp(s[j]) for j in vis)
        for c in range(v.shape[1]):
            o[i, c] = float(mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(v[j, c]) for j in vis) / z)
        lse[i] = float(mpmath.log(z))
    return o, lse


@pytest.mark.parametrize("nq,nkv,dqk,dv,causal", [
    (1, 1, 1, 1, False), (3, 5, 2, 3, False), (5, 3, 4, 2, True), (4, 4, 3, 5, True),
    (2, 7, 8, 8, True), (8, 8, 8, 4, False), (7, 2, 2, 2, True),
])
@pytest.mark.parametrize("scale", [0.7, -0.45])
def test_brute_force_tiny(nq, nkv, dqk, dv, causal, scale):
    rng = np.random.default_rng(nq * 100 + nkv * 10 + dqk + causal)
    q, k, v = rng.standard_normal((nq, dqk)) * 2, rng.standard_normal((nkv, dqk)), rng.standard_normal((nkv, dv))
    o, lse = oracle.head(q, k, v, scale, causal)
    ob, lb = brute_force(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    assert np.array_equal(np.isfinite(lse), fin)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    n, d, dv, scale = 37, 16, 12, 0.3
    q, v = rand(n, d), rand(n, dv)
    kvec = rand(d)
    k = np.tile(kvec, (n, 1))
    o, lse = oracle.head(q, k, v, scale, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - (scale * q[i] @ kvec + math.log(cnt))) < 1e-12


def test_single_key_returns_its_value():
    q, k, v = rand(9, 8), rand(1, 8), rand(1, 5)
    o, lse = oracle.head(q, k, v, 0.5, False)
    np.testing.assert_array_equal(o, np.tile(v[0], (9, 1)))
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]), atol=1e-14)


def test_rows_of_p_sum_to_one():
    q, k, v = rand(20, 8), rand(31, 8), rand(31, 4)
    scale = 1.3
    _, lse = oracle.head(q, k, v, scale, False)
    s = scale * np.einsum("id,jd->ij", q, k)
    np.testing.assert_allclose(np.exp(s - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)


def test_causal_first_row_is_first_value():
    q, k, v = rand(16, 8), rand(16, 8), rand(16, 6)
    o, lse = oracle.head(q, k, v, 0.4, True)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - 0.4 * q[0] @ k[0]) < 1e-14


def test_scale_zero_gives_uniform_average():
    q, k, v = rand(10, 4), rand(10, 4), rand(10, 3)
    o, lse = oracle.head(q, k, v, 0.0, True)
    for i in range(10):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(0), atol=1e-14)
        assert abs(lse[i] - math.log(i + 1)) < 1e-14


def test_two_keys_sigmoid_form():
    q, k, v = rand(6, 3), rand(2, 3), rand(2, 4)
    scale = 0.9
    o, lse = oracle.head(q, k, v, scale, False)
    s0, s1 = scale * q @ k[0], scale * q @ k[1]
    w0 = 1.0 / (1.0 + np.exp(s1 - s0))
    np.testing.assert_allclose(o, w0[:, None] * v[0] + (1 - w0)[:, None] * v[1], atol=1e-14)
    np.testing.assert_allclose(lse, np.logaddexp(s0, s1), atol=1e-14)


def test_negative_scale_prefers_the_smallest_score():
    # A negative scale reverses the ordering of the scores: with scale -1 and
    # scores q.k of ln 3 and 0, the weights are exp(-ln 3) : 1 = 1/4 : 3/4.
    q = np.array([[1.0]])
    k = np.array([[math.log(3.0)], [0.0]])
    v = np.array([[4.0, -8.0], [0.0, 8.0]])
    o, lse = oracle.head(q, k, v, -1.0, False)
    np.testing.assert_allclose(o[0], [1.0, 4.0], atol=1e-15)
    assert abs(lse[0] - math.log(4.0 / 3.0)) < 1e-15


def test_hand_worked_example():
    # Scores differ by ln 3, so the two weights are exactly 3/4 and 1/4.
    q = np.array([[1.0]])
    k = np.array([[math.log(3.0)], [0.0]])
    v = np.array([[4.0, -8.0], [0.0, 8.0]])
    o, lse = oracle.head(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0], [3.0, -4.0], atol=1e-15)
    assert abs(lse[0] - math.log(4.0)) < 1e-15


# ---------------------------------------------------------------- invariances
def test_value_affine_map():
    q, k, v = rand(12, 8), rand(15, 8), rand(15, 5)
    a, b = -2.5, rand(5)
    o, _ = oracle.head(q, k, v, 0.6, True)
    o2, _ = oracle.head(q, k, a * v + b, 0.6, True)
    np.testing.assert_allclose(o2, a * o + b, atol=1e-12)


def test_key_shift():
    q, k, v = rand(12, 8), rand(15, 8), rand(15, 5)
    u = rand(8)
    o, lse = oracle.head(q, k, v, 0.6, False)
    o2, lse2 = oracle.head(q, k + u, v, 0.6, False)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 0.6 * q @ u, atol=1e-12)


def test_permutations():
    q, k, v = rand(12, 8), rand(15, 8), rand(15, 5)
    o, lse = oracle.head(q, k, v, 0.6, False)
    pk = RNG.permutation(15)
    o2, lse2 = oracle.head(q, k[pk], v[pk], 0.6, False)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    pq = RNG.permutation(12)
    o3, lse3 = oracle.head(q[pq], k, v, 0.6, False)
    np.testing.assert_allclose(o3, o[pq], atol=1e-13)
    np.testing.assert_allclose(lse3, lse[pq], atol=1e-13)


def test_causal_ignores_future_keys():
    q, k, v = rand(20, 8), rand(20, 8), rand(20, 5)
    o, lse = oracle.head(q, k, v, 0.6, True)
    k2, v2 = k.copy(), v.copy()
    k2[11:] = rand(9, 8) * 5
    v2[11:] = rand(9, 5) * 5
    o2, lse2 = oracle.head(q, k2, v2, 0.6, True)
    np.testing.assert_array_equal(o2[:11], o[:11])
    np.testing.assert_array_equal(lse2[:11], lse[:11])
    assert not np.allclose(o2[11:], o[11:])


def test_causal_alignment_bottom_right():
    # N_q < N_kv: the last query sees every key, the first sees N_kv - N_q + 1.
    q, k, v = rand(5, 8), rand(12, 8), rand(12, 5)
    oc, lc = oracle.head(q, k, v, 0.6, True)
    on, ln_ = oracle.head(q, k, v, 0.6, False)
    np.testing.assert_allclose(oc[-1], on[-1], atol=1e-14)
    o_first, l_first = oracle.head(q[:1], k[:8], v[:8], 0.6, False)
    np.testing.assert_allclose(oc[0], o_first[0], atol=1e-14)
    # N_q > N_kv: the first N_q - N_kv rows see no key at all.
    q, k, v = rand(9, 4), rand(4, 4), rand(4, 3)
    o, lse = oracle.head(q, k, v, 1.0, True)
    np.testing.assert_array_equal(o[:5], 0.0)
    assert np.all(np.isneginf(lse[:5]))
    np.testing.assert_array_equal(o[5], v[0])


def test_large_logits_are_stable():
    q, k, v = rand(6, 4), rand(9, 4), rand(9, 3)
    o, lse = oracle.head(q * 1e3, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s = 1e3 * q @ k.T
    top2 = np.sort(s, axis=1)[:, -2:]
    clear = top2[:, 1] - top2[:, 0] > 60.0       # exp(-60) is far below 1e-10
    assert clear.sum() >= 3
    np.testing.assert_allclose(o[clear], v[np.argmax(s, axis=1)][clear], atol=1e-10)
    np.testing.assert_allclose(lse[clear], s.max(axis=1)[clear], atol=1e-9)


def test_rotation_invariance():
    d = 128
    q, k, v = rand(33, d), rand(40, d), rand(40, 16)
    r = oracle.rotation(RNG.choice([-1.0, 1.0], size=d))
    o, lse = oracle.head(q, k, v, d ** -0.5, True)
    o2, lse2 = oracle.head(q @ r, k @ r, v, d ** -0.5, True)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


# ---------------------------------------------------------------- plumbing
def test_batched_chunked_and_sampled_agree():
    import torch

    g = torch.Generator().manual_seed(7)
    q = torch.randn(2, 3, 50, 16, generator=g).to(torch.bfloat16)
    k = torch.randn(2, 3, 61, 16, generator=g).to(torch.bfloat16)
    v = torch.randn(2, 3, 61, 8, generator=g).to(torch.bfloat16)
    o, lse = oracle.attention(q, k, v, 0.25, True)
    qf = oracle.to_f64(q)
    assert qf.dtype == np.float64 and np.array_equal(qf, q.float().numpy())
    # Different row chunks may take a different BLAS blocking: last-bit differences only.
    oc, lc = oracle.head(q[1, 2], k[1, 2], v[1, 2], 0.25, True, max_bytes=8 * 61 * 7)
    np.testing.assert_allclose(oc, o[1, 2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lc, lse[1, 2], rtol=0, atol=1e-14)
    os_, ls_ = oracle.attention_rows(q, k, v, 0.25, True, [(0, 1, 0), (1, 2, 49), (1, 0, 13)])
    for n, (b, h, i) in enumerate([(0, 1, 0), (1, 2, 49), (1, 0, 13)]):
        np.testing.assert_allclose(os_[n], o[b, h, i], rtol=0, atol=1e-14)
        assert abs(ls_[n] - lse[b, h, i]) < 1e-14
    op, lp = oracle.attention_parallel(q, k, v, 0.25, True, processes=2)
    np.testing.assert_allclose(op, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lp, lse, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- mutation check
def _pins_fail(head_fn):
    """Run a subset of the closed-form pins against ``head_fn``; count failures."""
    fails = 0
    rng = np.random.default_rng(99)
    # identical keys, causal, scale != 1, N_q < N_kv
    q, v = rng.standard_normal((6, 5)), rng.standard_normal((9, 3))
    kvec = rng.standard_normal(5)
    k = np.tile(kvec, (9, 1))
    o, lse = head_fn(q, k, v, 0.37, True)
    for i in range(6):
        cnt = i + 1 + 3
        if not np.allclose(o[i], v[:cnt].mean(0), atol=1e-12):
            fails += 1
        if abs(lse[i] - (0.37 * q[i] @ kvec + math.log(cnt))) > 1e-12:
            fails += 1
    # two keys, asymmetric dims
    q, k, v = rng.standard_normal((4, 3)), rng.standard_normal((2, 3)), rng.standard_normal((2, 5))
    o, lse = head_fn(q, k, v, 0.9, False)
    s0, s1 = 0.9 * q @ k[0], 0.9 * q @ k[1]
    w0 = 1.0 / (1.0 + np.exp(s1 - s0))
    if not np.allclose(o, w0[:, None] * v[0] + (1 - w0)[:, None] * v[1], atol=1e-12):
        fails += 1
    if not np.allclose(lse, np.logaddexp(s0, s1), atol=1e-12):
        fails += 1
    return fails


def _mutant(kind):
    def head_fn(qh, kh, vh, scale, causal):
        qh, kh, vh = map(np.asarray, (qh, kh, vh))
        n_q, n_kv = qh.shape[0], kh.shape[0]
        sc = 1.0 if kind == "drop_scale" else scale
        s = sc * (qh @ kh.T)
        if kind == "sign":
            s = -s
        if causal:
            off = 0 if kind == "top_left_causal" else n_kv - n_q
            j = np.arange(n_kv)[None, :]
            s = np.where(j > np.arange(n_q)[:, None] + off, -np.inf, s)
        m = s.max(1)
        p = np.exp(s - m[:, None])
        l = p.sum(1)
        if kind == "no_normalise":
            l = np.ones_like(l)
        o = p @ vh / l[:, None]
        lse = m + (np.log2(l) if kind == "log2_lse" else np.log(l))
        if kind == "lse_without_max":
            lse = np.log(l)
        return o, lse
    return head_fn


@pytest.mark.parametrize("kind", ["drop_scale", "sign", "top_left_causal", "no_normalise",
                                  "log2_lse", "lse_without_max"])
def test_pins_catch_planted_mistakes(kind):
    assert _pins_fail(lambda *a: oracle.head(*a)) == 0
    assert _pins_fail(_mutant(kind)) > 0
