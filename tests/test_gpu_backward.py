"""GPU parity of attn_bwd (dQ, dK, dV) against the float64 gradient oracle.

Tolerance (a reading; the pages give none for the backward pass): each gradient is a
sum of products whose operands are bf16 (fp16) values with fp32 accumulation, and the
softmax weights P and dS are rounded to 16 bits before their products (relative
error 2^-9 each), the output once more (2^-9). The gate is a relative Frobenius error
of at most 1e-2 per gradient tensor (about 2.5 x 2^-8) and, per element,
|error| <= 2e-2 * max|reference| + 2^-7 |reference|.
"""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import f64, log, record, to_dev

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2


def gate(got, ref, label):
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    worst = float((err / (2e-2 * scale + 2.0 ** -7 * np.abs(ref) + 1e-30)).max())
    log(f"{label}: rel Frobenius {fro:.3e}, max abs {err.max():.3e} (max |ref| {scale:.3e}), "
        f"worst err/bound {worst:.3f}")
    record(label, dict(rel_frobenius=float(fro), max_abs=float(err.max()), max_ref=float(scale),
                       worst_over_bound=worst))
    assert np.all(np.isfinite(got)), f"{label}: non-finite gradient"
    assert fro <= REL_FRO, f"{label}: relative Frobenius error {fro}"
    assert worst <= 1.0, f"{label}: elementwise error {worst}"


def run_case(B, H, nq, nkv, d, causal, seed, dtype=torch.bfloat16, scale=None):
    scale = d ** -0.5 if scale is None else scale
    label = f"bwd B{B} H{H} Nq{nq} Nkv{nkv} d{d} causal={causal} {dtype} scale={scale:.4f} seed={seed}"
    log("start " + label)
    q, k, v = synth.qkv(B, H, nq, nkv, d, d, seed, dtype)
    g = torch.Generator("cpu").manual_seed(seed + 1)
    do = torch.randn((B, H, nq, d), generator=g, dtype=torch.float32).to(dtype)
    dq_, dk_, dv_, ddo = to_dev(q, k, v, do)
    o, lse = ea.attn_fwd(dq_, dk_, dv_, causal=causal, scale=scale)
    gq, gk, gv = ea.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    for name, got, ref in (("dQ", gq, rq), ("dK", gk, rk), ("dV", gv, rv)):
        gate(f64(got), ref, f"{label} {name}")
    return gq, gk, gv


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 128, 128, 64), (2, 3, 300, 300, 128), (2, 2, 100, 333, 128),
                                   (1, 2, 257, 129, 64), (1, 4, 1024, 1024, 128), (1, 1, 1, 1, 64),
                                   (2, 2, 31, 95, 64), (1, 2, 700, 300, 128), (1, 2, 300, 700, 128)],
                         ids=lambda s: "B{}H{}_{}x{}_d{}".format(*s))
def test_backward(shape, causal):
    B, H, nq, nkv, d = shape
    run_case(B, H, nq, nkv, d, causal, seed=3000 + nq + nkv + d + int(causal))


def test_backward_fp16():
    run_case(2, 2, 200, 260, 128, True, seed=3101, dtype=torch.float16)
    run_case(1, 3, 150, 150, 64, False, seed=3102, dtype=torch.float16)


def test_backward_deterministic_and_empty_rows():
    q, k, v = synth.qkv(1, 2, 64, 20, 64, 64, seed=3201)
    g = torch.Generator("cpu").manual_seed(3202)
    do = torch.randn((1, 2, 64, 64), generator=g).to(torch.bfloat16)
    dq_, dk_, dv_, ddo = to_dev(q, k, v, do)
    log("start bwd determinism / empty rows")
    o, lse = ea.attn_fwd(dq_, dk_, dv_, causal=True)
    a = ea.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=True)
    b = ea.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # causal with N_q = 64 > N_kv = 20: queries 0..43 see no key and get dQ = 0
    assert torch.all(a[0][:, :, :44] == 0)


def _sampled_heads(B, H, n, d, causal, seed, heads):
    """Full-size launch; the oracle computes the gradients of a few whole heads."""
    label = f"bwd B{B} H{H} N{n} d{d} causal={causal} heads {heads}"
    log("start " + label)
    q, k, v = synth.qkv(B, H, n, n, d, d, seed)
    g = torch.Generator("cpu").manual_seed(seed + 1)
    do = torch.randn((B, H, n, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    dq_, dk_, dv_, ddo = to_dev(q, k, v, do)
    o, lse = ea.attn_fwd(dq_, dk_, dv_, causal=causal)
    gq, gk, gv = ea.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=causal)
    torch.cuda.synchronize()
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv, _ = oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], d ** -0.5, causal)
        for name, got, ref in (("dQ", gq, rq), ("dK", gk, rk), ("dV", gv, rv)):
            gate(f64(got[sl]), ref, f"{label} ({b},{h}) {name}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_benchmark_shape(causal):
    """B4 H16 N2048 d128, the benchmarked backward workload, on two sampled heads."""
    _sampled_heads(4, 16, 2048, 128, causal, seed=3301 + int(causal), heads=[(0, 0), (3, 15)])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_many_items(causal):
    """576 workgroups per kernel (more than the 256 compute units), heavy and light
    causal tiles mixed; every head checked."""
    run_case(2, 72, 512, 512, 128, causal, seed=3401 + int(causal))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_negative_scale(causal):
    run_case(2, 3, 300, 300, 128, causal, seed=3301 + int(causal), scale=-128 ** -0.5)
    run_case(1, 2, 100, 257, 64, causal, seed=3311 + int(causal), scale=-0.3)
