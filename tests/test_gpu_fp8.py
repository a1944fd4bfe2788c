"""GPU parity of the fp8 path: the quantiser bit-exact against the oracle's
codec, and the fp8 attention forward against the float64 oracle."""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import f64, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("N", [128, 400, 1024])
def test_quantize_bit_exact(rotate, transpose, N):
    log(f"start quantize N={N} rotate={rotate} transpose={transpose}")
    signs, q, _, _ = synth.fp8_inputs(2, 3, N, 128, seed=N + 7)
    dx, ds = to_dev(q, signs)
    x8, desc = ea.attn_quantize_fp8(dx, signs=ds if rotate else None, transpose=transpose)
    torch.cuda.synchronize()
    codes, d_ref = oracle.quantize_blocks(q, signs.numpy() if rotate else None)
    got = x8.cpu().numpy()
    if transpose:
        got = np.swapaxes(got, 2, 3)
    mism = int((got != codes).sum())
    log(f"  code mismatches {mism} of {codes.size}")
    assert mism == 0
    assert np.array_equal(desc.cpu().numpy(), d_ref)


def test_quantize_config5_full():
    w = synth.workload("fp8")
    log(f"start quantize {w.label()}")
    signs, q, k, v = synth.fp8_inputs(w.B, w.H, w.N_q, w.d_qk, w.seed)
    dq, dk, dv, ds = to_dev(q, k, v, signs)
    for name, x, dx, sg, tr in (("q", q, dq, ds, False), ("k", k, dk, ds, False), ("v", v, dv, None, True)):
        x8, desc = ea.attn_quantize_fp8(dx, signs=sg, transpose=tr)
        torch.cuda.synchronize()
        codes, d_ref = oracle.quantize_blocks(x, signs.numpy() if sg is not None else None)
        got = x8.cpu().numpy()
        if tr:
            got = np.swapaxes(got, 2, 3)
        mism = int((got != codes).sum())
        log(f"  {name}: code mismatches {mism} of {codes.size}")
        assert mism == 0
        assert np.array_equal(desc.cpu().numpy(), d_ref)


# ---------------------------------------------------------------- fp8 attention
#
# What the kernel consumes is fixed by the oracle's codec: Q, K (rotated or not)
# and V are quantised on the host by oracle.quantize_blocks; the GPU quantiser's
# codes must equal them bit for bit, and the expected values come from the oracle
# alone.
#
# Bound against the oracle on the dequantised inputs (Q^, K^, V^).
#
# Scores. v_mfma_f32_32x32x64_f8f6f4 does not sum its 64 products exactly: a
# host-checked probe of the instruction on random e4m3 operands (N(0,1), x30
# outliers, one dominant product) found errors up to 2^-11.5 of the largest
# product of the sum. With eps = 2^-10 per product (a margin over that), the
# two K-steps of a score give |dS_ij| <= 2 eps scale |q^_i|_max |k^_j|_max,
# hence delta_i = 2^-9 scale |q^_i|_max max_j |k^_j|_max bounds the score
# error of row i, and LSE_i moves by at most delta_i (plus float32 rounding,
# 1e-3). Perturbing every score of a row by at most delta_i moves each
# softmax weight by a factor within e^(+-2 delta_i).
#
# P -> e4m3: a normal e4m3 value is within 2^-4 of p (relative), a subnormal one
# within 2^-10 in the kernel's p units, where a row's largest p is at least 2^6
# and the p of a tile carries the factor dv_tile / dv_max of its V descale.
#
# Hence, per element, with P the oracle's softmax and A_i = sum_j P_ij |v^_j|,
#   |dO_i| <= (2^-4 + e^(2 delta_i) - 1) A_i + 2^-16 sum_j |v^_j| dv_max / dv_j
#             + 2^-8 |O_i| (bf16 output) + 1e-4.
# The elementwise bound is a worst case (every error of a row with the same
# sign). Errors of independent keys largely cancel: a host model of a kernel
# that only rounds P to e4m3 stays at 2-4 % of mean |O| in mean absolute error
# on N(0,1) inputs, so the mean error is also gated at 10 % of mean |O|; a
# kernel that pairs P with the wrong keys misses that by far.

def _fp8_case(q, k, v, signs, rotate, scale, causal, label):
    sg = signs.numpy() if rotate else None
    ref = {name: oracle.quantize_blocks(x, sg if name != "v" else None)
           for name, x in (("q", q), ("k", k), ("v", v))}
    dq_, dk_, dv_, ds = to_dev(q, k, v, signs)
    g = {}
    for name, dx in (("q", dq_), ("k", dk_), ("v", dv_)):
        tr = name == "v"
        x8, desc = ea.attn_quantize_fp8(dx, signs=(ds if rotate and not tr else None), transpose=tr)
        got = x8.cpu().numpy()
        if tr:
            got = np.swapaxes(got, 2, 3)
        assert np.array_equal(got, ref[name][0]), f"{label}: {name} codes differ from the oracle's"
        assert np.array_equal(desc.cpu().numpy(), ref[name][1])
        g[name] = (x8, desc)
    o, lse = ea.attn_fwd_fp8(g["q"][0], g["k"][0], g["v"][0], g["q"][1], g["k"][1], g["v"][1],
                             causal=causal, scale=scale)
    torch.cuda.synchronize()
    deq = {n: oracle.dequantize_blocks(*ref[n]) for n in ref}
    return f64(o), f64(lse), deq, ref


def _score_delta(deq, scale):
    """delta_i [B,H,N_q,1]: bound on the score error of row i."""
    qmax = np.abs(deq["q"]).max(axis=3, keepdims=True)
    kmax = np.abs(deq["k"]).max(axis=(2, 3), keepdims=True)
    return 2.0 ** -9 * scale * qmax * kmax


def _fp8_bound(deq, ref, scale, causal, oracle_fn=None):
    qh, kh, vh = deq["q"], deq["k"], deq["v"]
    fn = oracle_fn or oracle.attention
    o_ref, lse_ref = fn(qh, kh, vh, scale, causal)
    o_abs, _ = fn(qh, kh, np.abs(vh), scale, causal)
    dv = np.asarray(ref["v"][1], dtype=np.float64)                      # [B,H,nb]
    dv_max = dv.max(axis=2, keepdims=True)
    w = np.where(dv > 0, dv_max / np.where(dv > 0, dv, 1.0), 1.0)       # dv_max / dv_j
    N = vh.shape[2]
    wt = np.repeat(w, oracle.BLOCK_TOKENS, axis=2)[:, :, :N, None]
    sub = (np.abs(vh) * wt).sum(axis=2, keepdims=True)                   # [B,H,1,d]
    delta = _score_delta(deq, scale)
    bound = ((2.0 ** -4 + np.expm1(2 * delta)) * o_abs + 2.0 ** -16 * sub
             + 2.0 ** -8 * np.abs(o_ref) + 1e-4)
    return o_ref, lse_ref, bound, 1e-3 + delta[..., 0]


def _gate_fp8(o, lse, o_ref, lse_ref, bound, lse_tol, label, mean_gate=True):
    assert np.all(np.isfinite(o)), f"{label}: non-finite O"
    err = np.abs(o - o_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{label}: LSE finiteness differs"
    assert np.all(lse[~fin] == lse_ref[~fin])
    dl = np.where(fin, np.abs(np.where(fin, lse, 0) - np.where(fin, lse_ref, 0)), 0.0)
    mean_o = float(np.abs(o_ref).mean())
    log(f"{label}: vs dequantised oracle O max abs {err.max():.3e}, mean abs {err.mean():.3e} "
        f"({err.mean() / mean_o:.4f} of mean |O|), worst err/bound {(err / bound).max():.3f}; "
        f"LSE max abs {dl.max():.3e}, worst LSE err/bound {(dl / lse_tol).max():.3f}")
    assert (err / bound).max() <= 1.0, f"{label}: elementwise fp8 bound failed"
    assert (dl <= lse_tol).all(), f"{label}: LSE bound failed"
    if mean_gate:
        assert err.mean() <= 0.1 * mean_o, f"{label}: mean fp8 error gate failed"
    return float(err.mean())


FP8_SHAPES = [  # (B, H, N_q, N_kv, causal)
    (1, 2, 256, 256, False),
    (1, 2, 256, 256, True),
    (2, 3, 300, 400, False),
    (2, 3, 300, 400, True),
    (1, 2, 129, 1040, False),
    (1, 2, 129, 1040, True),
    (1, 1, 700, 96, True),      # N_q > N_kv: the first 604 rows see no key
    (1, 2, 1024, 2048, False),
]


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "B{}H{}q{}kv{}{}".format(*s[:4], "c" if s[4] else ""))
def test_fp8_attention_parity(shape, rotate):
    B, H, nq, nkv, causal = shape
    label = f"fp8 B{B} H{H} Nq{nq} Nkv{nkv} causal={causal} rotate={rotate}"
    log(f"start {label}")
    signs, q, _, _ = synth.fp8_inputs(B, H, nq, 128, seed=nq + 3, outlier_frac=0.0)
    _, _, k, v = synth.fp8_inputs(B, H, nkv, 128, seed=nkv + 5, outlier_frac=0.0)
    scale = 128 ** -0.5
    o, lse, deq, ref = _fp8_case(q, k, v, signs, rotate, scale, causal, label)
    o_ref, lse_ref, bound, lse_tol = _fp8_bound(deq, ref, scale, causal)
    _gate_fp8(o, lse, o_ref, lse_ref, bound, lse_tol, label)


def test_fp8_attention_zero_blocks():
    """An all-zero V block (descale 0) and an all-zero K block still count in l."""
    label = "fp8 zero blocks"
    log(f"start {label}")
    signs, q, k, v = synth.fp8_inputs(1, 2, 512, 128, seed=77, outlier_frac=0.0)
    v[:, :, 128:256] = 0
    k[:, 1, 256:384] = 0
    scale = 128 ** -0.5
    o, lse, deq, ref = _fp8_case(q, k, v, signs, True, scale, False, label)
    assert (ref["v"][1][:, :, 1] == 0).all()
    o_ref, lse_ref, bound, lse_tol = _fp8_bound(deq, ref, scale, False)
    _gate_fp8(o, lse, o_ref, lse_ref, bound, lse_tol, label)


def _errors(o, o_ref):
    e = o - o_ref
    return dict(max_abs=float(np.abs(e).max()), mean_abs=float(np.abs(e).mean()),
                rmse=float(np.sqrt((e * e).mean())))


def test_fp8_config5_outlier_free():
    """Outlier-free N(0,1) inputs at the fp8 workload's shape: max abs <= 6e-2
    against the oracle on the original bfloat16 inputs, rotated and not."""
    w = synth.workload("fp8")
    signs, q, k, v = synth.fp8_inputs(w.B, w.H, w.N_q, w.d_qk, w.seed, outlier_frac=0.0)
    o_orig, lse_orig = oracle.attention_parallel(q, k, v, w.scale, False, processes=16)
    for rotate in (False, True):
        label = f"fp8 {w.label()} outlier-free rotate={rotate}"
        log(f"start {label}")
        o, lse, _, _ = _fp8_case(q, k, v, signs, rotate, w.scale, False, label)
        st = _errors(o, o_orig)
        dl = float(np.abs(lse - lse_orig).max())
        log(f"{label}: vs original O max abs {st['max_abs']:.3e} (gate 6e-2), mean abs "
            f"{st['mean_abs']:.3e}, RMSE {st['rmse']:.3e}; LSE max abs {dl:.3e}")
        assert st["max_abs"] <= 6e-2


def test_fp8_config5_outliers():
    """The fp8 workload as stated (0.5 % of coordinates x30). Against the oracle
    on the dequantised inputs: the elementwise bound above, rotated and not; the
    mean error is reported. (An error-free kernel that only rounds P to e4m3
    reaches a mean abs of about 2.7e-3 here; the x30 outliers raise the block
    amax of Q and K, and with it the MFMA's summation error on every score, which
    takes the measured mean abs to about 1.7e-2.) Against the original inputs:
    rotated mean abs <= 6e-2 and a lower RMSE than without rotation; both errors
    and their ratio are reported."""
    w = synth.workload("fp8")
    signs, q, k, v = synth.fp8_inputs(w.B, w.H, w.N_q, w.d_qk, w.seed)
    par = lambda *a: oracle.attention_parallel(*a, processes=16)
    o_orig, _ = par(q, k, v, w.scale, False)
    res = {}
    for rotate in (False, True):
        label = f"fp8 {w.label()} rotate={rotate}"
        log(f"start {label}")
        o, lse, deq, ref = _fp8_case(q, k, v, signs, rotate, w.scale, False, label)
        o_deq, lse_deq, bound, lse_tol = _fp8_bound(deq, ref, w.scale, False, oracle_fn=par)
        mean_deq = _gate_fp8(o, lse, o_deq, lse_deq, bound, lse_tol, label, mean_gate=False)
        so = _errors(o, o_orig)
        log(f"{label}: vs original O max abs {so['max_abs']:.3e}, mean abs {so['mean_abs']:.3e}, "
            f"RMSE {so['rmse']:.3e}")
        log(f"{label}: mean abs vs dequantised {mean_deq:.3e}")
        res[rotate] = so
    log(f"fp8 rotation: RMSE unrotated/rotated = {res[False]['rmse'] / res[True]['rmse']:.2f}, "
        f"mean abs ratio {res[False]['mean_abs'] / res[True]['mean_abs']:.2f}")
    assert res[True]["mean_abs"] <= 6e-2
    assert res[True]["rmse"] < res[False]["rmse"]
