"""Pins for the grouped-query attention and split-merge oracle (oracle/decode.py).

The head grouping is a reading (consecutive query heads share a KV head); it is
pinned by a closed form that tells it apart from the other plausible order. The
merge is pinned against the full attention of the same inputs, which is an
independent evaluation of the same definition, over many ways of cutting the key
sequence (empty parts, parts a causal row cannot see, a single part).
"""
import numpy as np
import pytest

import oracle
from oracle import decode as odec

RNG = np.random.default_rng(777)


def rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- head grouping
def test_grouping_closed_form_identical_keys():
    """Identical keys give the plain mean of that KV head's values (uniform softmax).

    With H = 4 and H_kv = 2, heads 0 and 1 must return KV head 0's mean and heads
    2 and 3 KV head 1's; the interleaved order h % H_kv would give 0, 1, 0, 1.
    """
    B, H, H_kv, nq, nkv, d = 1, 4, 2, 3, 5, 8
    q = rand(B, H, nq, d)
    k = np.repeat(rand(B, H_kv, 1, d), nkv, axis=2)
    v = rand(B, H_kv, nkv, d)
    o, lse = oracle.attention_gqa(q, k, v, 0.7, causal=False)
    for h in range(H):
        g = h // 2
        np.testing.assert_allclose(o[0, h], np.broadcast_to(v[0, g].mean(axis=0), (nq, d)),
                                   rtol=0, atol=1e-13)
        s = 0.7 * q[0, h] @ k[0, g, 0]
        np.testing.assert_allclose(lse[0, h], s + np.log(nkv), rtol=0, atol=1e-12)


def test_mqa_is_broadcast_and_mha_is_identity():
    B, H, nq, nkv, d = 2, 6, 4, 9, 16
    q = rand(B, H, nq, d)
    k1, v1 = rand(B, 1, nkv, d), rand(B, 1, nkv, d)
    o, lse = oracle.attention_gqa(q, k1, v1, 0.3, causal=True)
    o_ref, lse_ref = oracle.attention(q, np.repeat(k1, H, axis=1), np.repeat(v1, H, axis=1),
                                      0.3, causal=True)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)
    kh, vh = rand(B, H, nkv, d), rand(B, H, nkv, d)
    o, lse = oracle.attention_gqa(q, kh, vh, 0.3)
    o_ref, lse_ref = oracle.attention(q, kh, vh, 0.3)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)


def test_kv_head_rule():
    assert [odec.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [odec.kv_head(h, 6, 6) for h in range(6)] == list(range(6))
    assert [odec.kv_head(h, 5, 1) for h in range(5)] == [0] * 5
    with pytest.raises(ValueError):
        oracle.attention_gqa(rand(1, 6, 2, 4), rand(1, 4, 3, 4), rand(1, 4, 3, 4), 1.0)


# ---------------------------------------------------------------- split and merge
def _split_merge(qh, kh, vh, scale, causal, cuts):
    bounds = [0] + list(cuts) + [kh.shape[0]]
    parts = [odec.head_keys(qh, kh, vh, scale, causal, a, b) for a, b in zip(bounds, bounds[1:])]
    return odec.merge([p[0] for p in parts], [p[1] for p in parts])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nkv", [(1, 40), (3, 40), (7, 7), (12, 5), (40, 64)])
def test_merge_of_splits_equals_full(causal, nq, nkv):
    d = 8
    qh, kh, vh = rand(nq, d), rand(nkv, d), rand(nkv, d)
    o_ref, lse_ref = oracle.head(qh, kh, vh, 0.5, causal)
    for cuts in ([], [nkv // 2], [1, nkv - 1], [0, 0, nkv // 3, nkv], sorted(RNG.integers(0, nkv + 1, 5))):
        o, lse = _split_merge(qh, kh, vh, 0.5, causal, cuts)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse))
        np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
        assert np.all(o[~fin] == 0)


def test_merge_identity_empty_and_associative():
    nq, nkv, d = 6, 30, 4
    qh, kh, vh = rand(nq, d), rand(nkv, d), rand(nkv, d)
    a = odec.head_keys(qh, kh, vh, 1.0, False, 0, 10)
    b = odec.head_keys(qh, kh, vh, 1.0, False, 10, 21)
    c = odec.head_keys(qh, kh, vh, 1.0, False, 21, 30)
    empty = odec.head_keys(qh, kh, vh, 1.0, False, 30, 30)
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    one = odec.merge([a[0]], [a[1]])
    np.testing.assert_allclose(one[0], a[0], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(one[1], a[1])
    with_empty = odec.merge([a[0], empty[0]], [a[1], empty[1]])
    np.testing.assert_allclose(with_empty[0], a[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(with_empty[1], a[1], rtol=0, atol=1e-15)
    ab = odec.merge([a[0], b[0]], [a[1], b[1]])
    bc = odec.merge([b[0], c[0]], [b[1], c[1]])
    left = odec.merge([ab[0], c[0]], [ab[1], c[1]])
    right = odec.merge([a[0], bc[0]], [a[1], bc[1]])
    flat = odec.merge([a[0], b[0], c[0]], [a[1], b[1], c[1]])
    for x in (left, right):
        np.testing.assert_allclose(x[0], flat[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(x[1], flat[1], rtol=0, atol=1e-13)
    none = odec.merge([empty[0], empty[0]], [empty[1], empty[1]])
    assert np.all(none[0] == 0) and np.all(np.isneginf(none[1]))


def test_head_keys_whole_range_is_head():
    qh, kh, vh = rand(5, 8), rand(11, 8), rand(11, 8)
    for causal in (False, True):
        o, lse = odec.head_keys(qh, kh, vh, 0.9, causal, 0, 11)
        o_ref, lse_ref = oracle.head(qh, kh, vh, 0.9, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- planted mistakes
def _mutant_merge(kind):
    def merge(o_parts, lse_parts):
        m = np.max(np.stack(lse_parts), axis=0)
        if kind == "no_max_shift_sign":
            w = [np.exp(m - x) for x in lse_parts]
        else:
            w = [np.exp(x - m) for x in lse_parts]
        total = sum(w)
        o = sum(wi[..., None] * oi for wi, oi in zip(w, o_parts))
        if kind != "no_normalise":
            o = o / total[..., None]
        lse = m + np.log(total) if kind != "lse_is_max" else m
        return o, lse
    return merge


@pytest.mark.parametrize("kind", ["no_max_shift_sign", "no_normalise", "lse_is_max"])
def test_merge_pins_catch_planted_mistakes(kind):
    nq, nkv, d = 4, 20, 4
    qh, kh, vh = rand(nq, d), rand(nkv, d), rand(nkv, d)
    o_ref, lse_ref = oracle.head(qh, kh, vh, 1.0, False)
    parts = [odec.head_keys(qh, kh, vh, 1.0, False, a, b) for a, b in ((0, 7), (7, 20))]
    o, lse = _mutant_merge(kind)([p[0] for p in parts], [p[1] for p in parts])
    assert not (np.allclose(o, o_ref, atol=1e-9) and np.allclose(lse, lse_ref, atol=1e-9))
