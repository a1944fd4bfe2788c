"""GPU parity of the fp8 path: the quantiser bit-exact against the oracle's
codec, and the fp8 attention forward against the float64 oracle."""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import f64, log, record, to_dev

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
# The kernel's arithmetic is modelled step by step in tests/fp8_kernel_model.py,
# including how v_mfma_f32_32x32x64_f8f6f4 adds its 64 products: in 8 groups of 8
# consecutive k, each product aligned to the group's largest exponent sum E and
# truncated toward zero to a multiple of 2^(E-13) (test_mfma_group_truncation pins
# this on the GPU through attn_fwd_fp8). The bound below follows from that model.
#
# Scores. A group loses less than 7 * 2^-13 of its largest product, so the 16
# groups of a score give |dS_ij| < 7 * 2^-13 * scale * sum_g max_{k in g}|q^_ik k^_jk|
# <= 7 * 2^-13 * scale * (qg_i . kg_j), with qg_i, kg_j the 16 group maxima of |q^_i|
# and |k^_j|; delta_i = max_j of that bounds the score error of row i. Perturbing
# every score of a row by at most delta_i moves each weight by a factor within
# e^(+-2 delta_i), and LSE_i by at most delta_i.
#
# Weights. p is rounded to e4m3: within 2^-4 of p (relative) when normal, within
# 2^-10 in the kernel's p units when subnormal, where a row's largest p is at least
# 2^6 and the p of a tile carries the factor dv_tile / dv_max of its V descale; so,
# relative to the row sum L, key j's rounding error is at most 2^-4 w_j + s_j with
# s_j = 2^-16 dv_max / dv_j. The row sum l adds the rounded p themselves (the
# weights the PV product uses), so O = sum_j p~_j v_j / sum_j p~_j and, with
# rho = 2^-4 + sum_j s_j, A_i = sum_j w_ij |v^_j| and T_i = sum_j s_j |v^_j|,
#   |dO_i| <= (2^-4 A_i + T_i + rho A_i) / (1 - rho)          (rounded weights)
#             + (e^(2 delta_i) - 1 + 2^-8) A_i                (scores; the PV and
#                                                              row-sum truncation)
#             + 2^-8 |O_i| (bf16 output) + 1e-4,
#   |dLSE_i| <= -ln(1 - rho - 2^-9) + delta_i + 1e-3.
# The elementwise bound is a worst case (every error of a row with the same sign).
# Errors of independent keys largely cancel, so the mean error is gated too: at 10 %
# of mean |O| on N(0,1) inputs, and on the x30-outlier workload at 1e-2 (G8b; the
# model predicts about 4.4e-3 there). On that workload the GPU must also agree with
# the model itself, row by row.

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
    """delta_i [B,H,N_q,1]: bound on the score error of row i (groups of 8 dims)."""
    B, H, nq, d = deq["q"].shape
    qg = np.abs(deq["q"]).reshape(B, H, nq, d // 8, 8).max(axis=4)       # [B,H,N_q,16]
    kg = np.abs(deq["k"]).reshape(B, H, -1, d // 8, 8).max(axis=4)       # [B,H,N_kv,16]
    worst = np.einsum("bhig,bhjg->bhij", qg, kg).max(axis=3, keepdims=True)
    return 7.0 * 2.0 ** -13 * abs(scale) * worst


def _fp8_bound(deq, ref, scale, causal, oracle_fn=None):
    qh, kh, vh = deq["q"], deq["k"], deq["v"]
    fn = oracle_fn or oracle.attention
    o_ref, lse_ref = fn(qh, kh, vh, scale, causal)
    o_abs, _ = fn(qh, kh, np.abs(vh), scale, causal)                    # A_i
    dv = np.asarray(ref["v"][1], dtype=np.float64)                      # [B,H,nb]
    dv_max = dv.max(axis=2, keepdims=True)
    w = np.where(dv > 0, dv_max / np.where(dv > 0, dv, 1.0), 1.0)       # dv_max / dv_j
    N = vh.shape[2]
    s_j = 2.0 ** -16 * np.repeat(w, oracle.BLOCK_TOKENS, axis=2)[:, :, :N]   # [B,H,N]
    rho = 2.0 ** -4 + s_j.sum(axis=2)[:, :, None, None]                 # [B,H,1,1]
    t_i = (np.abs(vh) * s_j[..., None]).sum(axis=2, keepdims=True)      # [B,H,1,d]
    delta = _score_delta(deq, scale)
    bound = ((2.0 ** -4 * o_abs + t_i + rho * o_abs) / (1.0 - rho)
             + (np.expm1(2 * delta) + 2.0 ** -8) * o_abs
             + 2.0 ** -8 * np.abs(o_ref) + 1e-4)
    lse_tol = -np.log1p(-(rho[..., 0] + 2.0 ** -9)) + delta[..., 0] + 1e-3
    return o_ref, lse_ref, bound, lse_tol


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
    record(label, dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                       mean_abs_over_mean_o=float(err.mean() / mean_o),
                       worst_ratio=float((err / bound).max()), lse_max_abs=float(dl.max()),
                       elements=int(err.size)))
    assert (err / bound).max() <= 1.0, f"{label}: elementwise fp8 bound failed"
    assert (dl <= lse_tol).all(), f"{label}: LSE bound failed"
    if mean_gate is True:
        assert err.mean() <= 0.1 * mean_o, f"{label}: mean fp8 error gate failed"
    elif mean_gate:
        assert err.mean() <= mean_gate, f"{label}: mean fp8 error gate ({mean_gate}) failed"
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


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_negative_scale(causal):
    label = f"fp8 negative scale causal={causal}"
    log(f"start {label}")
    signs, q, k, v = synth.fp8_inputs(2, 2, 384, 128, seed=4401 + int(causal), outlier_frac=0.0)
    scale = -128 ** -0.5
    o, lse, deq, ref = _fp8_case(q, k, v, signs, True, scale, causal, label)
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
    """The fp8 workload as stated (0.5 % of coordinates x30).

    G8b, against the oracle on the dequantised inputs: the elementwise bound above and
    mean abs <= 1e-2, rotated and not. The kernel model (fp8_kernel_model) predicts a
    mean abs of about 4.4e-3 here; the GPU result must agree with the model row by row
    on sampled rows of three heads: their mean difference at most a tenth of the model's
    own mean error against the oracle, which shows that the model accounts for the
    kernel's error.
    G8c, against the original inputs: rotated mean abs <= 6e-2 and a lower RMSE than
    without rotation; both errors and their ratio are reported."""
    import fp8_kernel_model as fm

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
        mean_deq = _gate_fp8(o, lse, o_deq, lse_deq, bound, lse_tol, label, mean_gate=1e-2)
        # the model of the kernel's arithmetic on sampled rows
        rng = np.random.default_rng(7)
        d_gm, d_mo = [], []
        for b, h in ((0, 0), (1, 5), (3, 15)):
            rows = np.sort(rng.choice(w.N_q, 64, replace=False))
            o_m, _ = fm.head_rows(ref["q"][0][b, h], ref["k"][0][b, h], ref["v"][0][b, h],
                                  ref["q"][1][b, h], ref["k"][1][b, h], ref["v"][1][b, h],
                                  w.scale, rows)
            d_gm.append(np.abs(o[b, h][rows] - o_m))
            d_mo.append(np.abs(o_m - o_deq[b, h][rows]))
        d_gm, d_mo = np.concatenate(d_gm), np.concatenate(d_mo)
        log(f"{label}: model vs dequantised oracle mean abs {d_mo.mean():.3e}; GPU vs model mean "
            f"abs {d_gm.mean():.3e}, max {d_gm.max():.3e}")
        record(label + " kernel model", dict(model_mean_abs=float(d_mo.mean()),
                                             gpu_vs_model_mean_abs=float(d_gm.mean()),
                                             gpu_vs_model_max_abs=float(d_gm.max())))
        assert d_gm.mean() <= 0.1 * d_mo.mean(), f"{label}: GPU does not follow the kernel model"
        so = _errors(o, o_orig)
        log(f"{label}: vs original O max abs {so['max_abs']:.3e}, mean abs {so['mean_abs']:.3e}, "
            f"RMSE {so['rmse']:.3e}")
        log(f"{label}: mean abs vs dequantised {mean_deq:.3e}")
        record(label + " vs original", so)
        res[rotate] = so
    log(f"fp8 rotation: RMSE unrotated/rotated = {res[False]['rmse'] / res[True]['rmse']:.2f}, "
        f"mean abs ratio {res[False]['mean_abs'] / res[True]['mean_abs']:.2f}")
    assert res[True]["mean_abs"] <= 6e-2
    assert res[True]["rmse"] < res[False]["rmse"]


# ---------------------------------------------------------------- the e4m3 MFMA sums
def _mfma_model_sum(a_vals, b_vals):
    """Sum of one 64-product e4m3 MFMA step as the kernel model describes it (float64
    of the exact group-truncated sum; the combination is exact for these operands)."""
    import fp8_kernel_model as fm

    a = oracle.e4m3_encode(a_vals)
    b = oracle.e4m3_encode(b_vals)
    return float(fm.mfma_dot(a[None, :], b[None, :], np.zeros((1, 1)))[0, 0])


def test_mfma_group_truncation():
    """Pins the model of v_mfma_f32_32x32x64_f8f6f4 through attn_fwd_fp8 on crafted codes.

    Scores: one key with crafted codes and 15 zero keys, descales 1 and a small scale so
    that the crafted score dominates: the LSE of each query is its score. A large product
    (448 x 448, exponent sum 16) truncates the other products of its group of 8 to
    multiples of 2^3: small products in the same group vanish or are cut toward zero,
    the same products in another group survive. Values: 64 keys with equal scores (all
    P = 2^6) and crafted V columns; O is the mean of the column, summed by the same
    instruction, so +448 and -448 in one group of 8 erase a small value beside them."""
    dev = torch.device("cuda:0")
    d = 128
    def row(small_dims, q_small, k_small, big_dim=0):
        q_ = np.zeros(d); k_ = np.zeros(d)
        q_[big_dim] = 448.0; k_[big_dim] = 448.0
        q_[small_dims] = q_small; k_[small_dims] = k_small
        return q_, k_
    cases = [row(list(range(1, 8)), 1.0, 2.0),         # products 2 < 2^3 beside 448^2: lost
             row(list(range(8, 15)), 1.0, 2.0),        # same products in the next group: kept
             row(list(range(1, 8)), 4.0, 4.0),         # 16, a multiple of 8: kept
             row(list(range(1, 8)), 3.0, 4.0),         # 12 -> 8 (toward zero)
             row(list(range(1, 8)), -3.0, 4.0),        # -12 -> -8 (toward zero, not -16)
             row(list(range(65, 72)), 1.0, 2.0, 64),   # the second K-step, same rule
             row([1], 1.0, 3 * 2.0 ** -9),             # a subnormal k beside it: lost
             row(list(range(1, 8)), 0.0, 0.0)]         # the big product alone
    nq = 32
    # one head per case: every query of a head meets the crafted key 0
    H = len(cases)
    q8 = np.zeros((1, H, nq, d), np.uint8); k8 = np.zeros((1, H, 16, d), np.uint8)
    for h, (q_, k_) in enumerate(cases):
        q8[0, h, :] = oracle.e4m3_encode(q_)
        k8[0, h, 0] = oracle.e4m3_encode(k_)
    v8t = np.zeros((1, H, d, 16), np.uint8)
    ones = lambda n: torch.ones(n, dtype=torch.float32, device=dev)
    scale = 2.0 ** -12
    log("start MFMA group truncation (scores)")
    o, lse = ea.attn_fwd_fp8(torch.from_numpy(q8).to(dev), torch.from_numpy(k8).to(dev),
                             torch.from_numpy(v8t).to(dev), ones(H), ones(H), ones(H),
                             scale=scale)
    torch.cuda.synchronize()
    lse = f64(lse)[0, :, 0]
    for h, (q_, k_) in enumerate(cases):
        qc, kc = oracle.e4m3_decode(oracle.e4m3_encode(q_)), oracle.e4m3_decode(oracle.e4m3_encode(k_))
        exact = float((qc * kc).sum())
        model = _mfma_model_sum(qc[:64], kc[:64])
        model = model + _mfma_model_sum(qc[64:], kc[64:])
        got = lse[h] / scale
        log(f"  case {h}: exact {exact:.6f} model {model:.6f} GPU {got:.6f}")
        assert abs(got - model) <= 1e-5 * abs(model), (h, exact, model, got)
        if abs(exact - model) > 1e-4 * abs(model):  # the truncation is visible in the LSE
            assert abs(got - exact) > 1e-5 * abs(exact)
    log("start MFMA group truncation (values)")
    n = 64
    vcol = np.zeros((3, n))
    vcol[0, [0, 1]] = [448.0, -448.0]; vcol[0, 2:8] = 2.0 ** -6      # small ones lost
    vcol[1, [0, 1]] = [448.0, -448.0]; vcol[1, 8:14] = 2.0 ** -6     # other group: kept
    vcol[2, [0, 1]] = [448.0, -448.0]; vcol[2, 2:8] = 2.0 ** -5      # product 2: kept
    v8t = np.zeros((1, 1, d, n), np.uint8)
    v8t[0, 0, :3] = oracle.e4m3_encode(vcol)
    q8 = np.zeros((1, 1, 32, d), np.uint8); k8 = np.zeros((1, 1, n, d), np.uint8)
    o, lse = ea.attn_fwd_fp8(torch.from_numpy(q8).to(dev), torch.from_numpy(k8).to(dev),
                             torch.from_numpy(v8t).to(dev), ones(1), ones(1), ones(1),
                             scale=0.1)
    torch.cuda.synchronize()
    o = f64(o)[0, 0, 0]
    p = np.full(n, 64.0)                       # every weight 2^6
    for c in range(3):
        vc = oracle.e4m3_decode(oracle.e4m3_encode(vcol[c]))
        model = _mfma_model_sum(p, vc) / (64.0 * n)
        exact = float((p * vc).sum()) / (64.0 * n)
        want = float(torch.tensor(model).to(torch.bfloat16).double())
        log(f"  column {c}: exact {exact:.6e} model {model:.6e} GPU {o[c]:.6e}")
        assert o[c] == want, (c, exact, model, o[c])
    assert o[0] == 0.0 and o[1] > 0.0 and o[2] > 0.0
