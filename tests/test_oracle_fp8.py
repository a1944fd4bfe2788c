"""Pins for the oracle's e4m3 codec, Hadamard rotation and block quantisation."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[~np.isnan(oracle.e4m3_decode(c))]


def test_decode_all_codes_matches_library_cast():
    c = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(c)
    lib = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    fin = ~np.isnan(mine)
    assert np.array_equal(mine[fin], lib[fin])
    assert np.isnan(mine[[0x7F, 0xFF]]).all() and np.isnan(mine).sum() == 2


def test_format_points():
    pts = json.load(open(os.path.join(GOLDEN, "e4m3_format_points.json")))["points"]
    vals = np.array([p["value"] for p in pts])
    codes = oracle.e4m3_encode(vals)
    assert codes.tolist() == [p["code"] for p in pts]
    assert oracle.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_encode_roundtrip_every_code():
    c = _finite_codes()
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(c)), c)


def _nearest_brute(x):
    """Nearest finite code by exhaustive search over magnitudes; ties to the even code.

    The sign bit is copied from x, so a negative value that rounds to zero is -0.
    """
    c = np.arange(0x7F, dtype=np.uint8)          # the 127 finite non-negative codes
    vals = oracle.e4m3_decode(c)
    out = []
    for xi in x:
        a = min(abs(xi), 448.0)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:
            best = [b for b in best if c[b] % 2 == 0]
        code = int(c[best[0]])
        out.append(code | (0x80 if np.signbit(xi) else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(3000) * 30,
        rng.uniform(-0.02, 0.02, 2000),
        rng.uniform(-500, 500, 1000),
    ]).astype(np.float32).astype(np.float64)
    assert np.array_equal(oracle.e4m3_encode(x), _nearest_brute(x))


def test_midpoints_round_to_even():
    c = _finite_codes()
    pos = np.sort(oracle.e4m3_decode(c[c < 0x80]))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = oracle.e4m3_encode(mids)
    assert np.all(enc % 2 == 0)
    lib = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, lib)


def test_hadamard_and_rotation():
    np.testing.assert_array_equal(oracle.hadamard(1), [[1.0]])
    np.testing.assert_array_equal(oracle.hadamard(2), [[1.0, 1.0], [1.0, -1.0]])
    for n in (4, 16, 128):
        h = oracle.hadamard(n)
        assert set(np.unique(h)) == {-1.0, 1.0}
        np.testing.assert_array_equal(h @ h.T, n * np.eye(n))
    s = np.random.default_rng(0).choice([-1.0, 1.0], size=128)
    r = oracle.rotation(s)
    np.testing.assert_allclose(r @ r.T, np.eye(128), atol=1e-15)
    np.testing.assert_allclose(np.abs(r), 128 ** -0.5, rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.hadamard(12)


def _bf16_block(seed, B=1, H=2, N=300, d=128, outliers=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, H, N, d, generator=g)
    if outliers:
        m = torch.rand(B, H, N, d, generator=g) < 0.005
        x = torch.where(m, x * 30, x)
    return x.to(torch.bfloat16)


def test_rotation_golden_sign_then_hadamard():
    """Hand-derived d = 4 example (tests/golden/rotation_sign_hadamard_4.json): the signs
    act on x's coordinates before the Hadamard mixing, x R = x diag(sigma) H / sqrt(d).
    R R^T = I and |R_ij| = 1/sqrt(d) hold for H diag(sigma) too; this value does not."""
    with open(os.path.join(GOLDEN, "rotation_sign_hadamard_4.json")) as fh:
        g = json.load(fh)
    x = np.array(g["x"])
    sigma = np.array(g["sigma"])
    np.testing.assert_array_equal(x @ oracle.rotation(sigma), g["x_rotated"])
    assert not np.allclose(x @ oracle.rotation(sigma), g["x_rotated_other_order"])
    # the quantiser applies the same rotation (unnormalised) and rounds 336 to even 320
    xb = torch.tensor(x, dtype=torch.float32).view(1, 1, 1, 4).to(torch.bfloat16)
    codes, desc = oracle.quantize_blocks(xb, sigma)
    np.testing.assert_array_equal(oracle.e4m3_decode(codes).reshape(-1), g["quantised_values"])
    assert desc.reshape(-1)[0] == np.float32(g["descale"])
    np.testing.assert_allclose(oracle.dequantize_blocks(codes, desc).reshape(-1),
                               np.array(g["quantised_values"]) * np.float32(g["descale"]))


@pytest.mark.parametrize("rotate", [False, True])
def test_block_quantisation_bounds(rotate):
    x = _bf16_block(1)
    signs = np.random.default_rng(1).choice([-1.0, 1.0], size=128) if rotate else None
    codes, desc = oracle.quantize_blocks(x, signs)
    assert codes.shape == (1, 2, 300, 128) and desc.shape == (1, 2, 3)
    xf = oracle.to_f64(x)
    ref = xf @ oracle.rotation(signs) if rotate else xf
    deq = oracle.dequantize_blocks(codes, desc)
    vals = np.abs(oracle.e4m3_decode(codes))
    for i in range(3):
        sl = slice(128 * i, 128 * (i + 1))
        # the largest element of every block lands exactly on +-448
        assert vals[:, :, sl].max(axis=(2, 3)).tolist() == [[448.0, 448.0]]
        err = np.abs(deq[:, :, sl] - ref[:, :, sl])
        d = desc[:, :, i][:, :, None, None].astype(np.float64)
        half_q = np.maximum(vals[:, :, sl] * 2.0 ** -4, 2.0 ** -10)
        assert np.all(err <= d * half_q * (1 + 1e-6) + np.abs(ref[:, :, sl]) * 2e-7)


def test_quantised_codes_use_unnormalised_rotation_exactly():
    # The code of each element depends only on y = x diag(s) H and the block amax.
    x = _bf16_block(2, N=128)
    s = np.random.default_rng(2).choice([-1.0, 1.0], size=128)
    codes, desc = oracle.quantize_blocks(x, s)
    y = oracle.to_f64(x) @ (s[:, None] * oracle.hadamard(128))
    amax = np.abs(y).max(axis=(2, 3))
    want = oracle.e4m3_encode((y * (448.0 / amax)[:, :, None, None]).astype(np.float32))
    assert np.array_equal(codes, want)
    np.testing.assert_array_equal(desc[:, :, 0], (amax / (448.0 * np.sqrt(128.0))).astype(np.float32))


def test_zero_block():
    x = torch.zeros(1, 1, 130, 128, dtype=torch.bfloat16)
    x[0, 0, 129, 3] = 2.0
    codes, desc = oracle.quantize_blocks(x, None)
    assert np.all(codes[0, 0, :128] == 0) and desc[0, 0, 0] == 0.0
    assert codes[0, 0, 129, 3] == 0x7E and desc[0, 0, 1] == np.float32(2.0 / 448.0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rotation_reduces_attention_error_on_outliers(seed):
    """Rotated block quantisation gives a smaller attention-output error.

    For a floating-point format the per-element error of x itself hardly
    changes under rotation (its relative error is constant); what the rotation
    removes is the large score error when outliers of q and k fall on the same
    coordinate. The ratio is not compared with the pages' figure, whose input
    distribution is not stated.
    """
    q = _bf16_block(10 + seed, N=512)
    k = _bf16_block(20 + seed, N=512)
    v = _bf16_block(30 + seed, N=512)
    s = np.random.default_rng(seed).choice([-1.0, 1.0], size=128)
    sc = 128 ** -0.5
    o, _ = oracle.attention(q, k, v, sc)
    deq = lambda x, sg=None: oracle.dequantize_blocks(*oracle.quantize_blocks(x, sg))
    dv = deq(v)
    o_plain, _ = oracle.attention(deq(q), deq(k), dv, sc)
    o_rot, _ = oracle.attention(deq(q, s), deq(k, s), dv, sc)
    rmse = lambda a: np.sqrt(((a - o) ** 2).mean())
    assert rmse(o_rot) < rmse(o_plain)


def test_table2_ideal_bf16_rounding():
    """Rounding 2^x (x on [0,1)) from float64 to bfloat16 reproduces the printed row."""
    g = json.load(open(os.path.join(GOLDEN, "table2_ideal_bf16_rounding.json")))
    x = np.random.default_rng(0).uniform(0.0, 1.0, 4 * 1024 * 1024)
    exact = np.exp2(x)
    rounded = torch.from_numpy(exact).to(torch.bfloat16).to(torch.float64).numpy()
    rel = np.abs(rounded - exact) / exact
    assert abs(rel.max() - g["max_rel_err"]) < 0.006e-3
    assert abs(rel.mean() - g["mean_rel_err"]) < 0.006e-3
    # and the bound used by the output tolerance covers it
    assert rel.max() <= 2.0 ** -8
