"""GPU parity of attn_fwd_decode (split-KV, grouped KV heads) against the float64 oracle.

Every call goes through the C ABI (ctypes binding). The oracle evaluates grouped-
query attention with the full key sequence per row (oracle.attention_gqa), so a
split-and-merge result is checked against the unsplit definition.
"""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import compare, f64, log, to_dev

pytestmark = pytest.mark.gpu


def run_case(B, H, H_kv, nq, nkv, d, causal, seed, splits=0, dtype=torch.bfloat16, scale=None):
    q, k, v = synth.qkv_gqa(B, H, H_kv, nq, nkv, d, seed, dtype)
    used = ea.attn_decode_splits(B, H, H_kv, nq, nkv, d, splits)
    scale = d ** -0.5 if scale is None else scale
    label = (f"decode B{B} H{H} Hkv{H_kv} Nq{nq} Nkv{nkv} d{d} causal={causal} {dtype} "
             f"splits={splits}->{used} scale={scale:.4f} seed={seed}")
    log("start " + label)
    dq, dk, dv = to_dev(q, k, v)
    o, lse = ea.attn_fwd_decode(dq, dk, dv, causal=causal, num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_gqa(q, k, v, scale, causal)
    return compare(f64(o), f64(lse), o_ref, lse_ref, label)


# (B, H, H_kv, N_q, N_kv, d): one row block (<= 32 rows), two (<= 64), four (<= 128).
CASES = [
    (2, 8, 2, 1, 4096, 128),      # 4 rows per KV head
    (4, 8, 8, 1, 2048, 128),      # plain multi-head decode
    (1, 32, 1, 4, 3000, 128),     # multi-query, 128 rows
    (3, 16, 4, 8, 777, 64),       # 32 rows, ragged keys
    (2, 16, 2, 8, 1500, 128),     # 64 rows
    (2, 12, 3, 5, 1031, 64),      # 20 rows
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Hkv{}_q{}_kv{}_d{}".format(*c))
@pytest.mark.parametrize("causal", [False, True])
def test_decode_auto_splits(case, causal):
    B, H, H_kv, nq, nkv, d = case
    run_case(B, H, H_kv, nq, nkv, d, causal, seed=sum(case) + int(causal))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64, 256])
def test_decode_explicit_splits(splits):
    run_case(2, 8, 2, 2, 2500, 128, True, seed=500 + splits, splits=splits)


@pytest.mark.parametrize("nkv", [1, 31, 32, 33, 95])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_short_keys(nkv, d):
    run_case(2, 4, 2, 3, nkv, d, True, seed=600 + nkv + d, splits=4)
    run_case(2, 4, 2, 3, nkv, d, False, seed=700 + nkv + d)


def test_decode_rows_without_keys():
    """Causal with N_q > N_kv: queries t < N_q - N_kv see no key (O = 0, LSE = -inf)."""
    q, k, v = synth.qkv_gqa(1, 4, 2, 20, 10, 64, seed=801)
    dq, dk, dv = to_dev(q, k, v)
    for splits in (1, 3):
        log(f"start rows without keys splits={splits}")
        o, lse = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_gqa(q, k, v, 0.125, True)
        compare(f64(o), f64(lse), o_ref, lse_ref, f"rows without keys splits={splits}")
        assert torch.all(o[:, :, :10] == 0) and torch.all(torch.isneginf(lse[:, :, :10]))


def test_decode_fp16():
    run_case(2, 8, 2, 4, 1800, 128, True, seed=811, dtype=torch.float16)
    run_case(2, 8, 4, 1, 900, 64, False, seed=812, dtype=torch.float16, splits=5)


def test_decode_every_output_written_and_deterministic():
    q, k, v = synth.qkv_gqa(3, 8, 2, 3, 1234, 128, seed=821)
    dq, dk, dv = to_dev(q, k, v)
    out = torch.full((3, 8, 3, 128), float("nan"), dtype=torch.bfloat16, device=dq.device)
    lse = torch.full((3, 8, 3), float("nan"), dtype=torch.float32, device=dq.device)
    log("start decode NaN sentinel")
    o1, l1 = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=6, out=out, lse=lse)
    o2, l2 = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=6)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_matches_prefill_kernel_on_full_heads():
    """H_kv = H and one split: the decode path and attn_fwd compute the same function."""
    q, k, v = synth.qkv_gqa(2, 4, 4, 16, 700, 128, seed=831)
    dq, dk, dv = to_dev(q, k, v)
    log("start decode vs attn_fwd")
    o1, l1 = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=1)
    o2, l2 = ea.attn_fwd(dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_gqa(q, k, v, 128 ** -0.5, True)
    compare(f64(o1), f64(l1), o_ref, lse_ref, "decode path")
    compare(f64(o2), f64(l2), o_ref, lse_ref, "prefill path")


def test_decode_workload_sampled():
    """The benchmark's decode workload at full size, checked on a sample of heads."""
    w = synth.decode_workload()
    q, k, v = synth.qkv_gqa(w.B, w.H, w.H_kv, w.N_q, w.N_kv, w.d, w.seed)
    dq, dk, dv = to_dev(q, k, v)
    log(f"start {w.label()}")
    o, lse = ea.attn_fwd_decode(dq, dk, dv, causal=w.causal)
    torch.cuda.synchronize()
    o, lse = f64(o), f64(lse)
    g = w.H // w.H_kv
    picks = [(0, 0), (0, w.H - 1), (w.B - 1, 5), (w.B // 2, w.H // 2 + 1)]
    for b, h in picks:
        o_ref, lse_ref = oracle.head(q[b, h], k[b, h // g], v[b, h // g], w.scale, w.causal)
        compare(o[b, h], lse[b, h], o_ref, lse_ref, f"{w.label()} head ({b},{h})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("splits", [1, 0, 5])
def test_decode_negative_scale(splits):
    run_case(2, 16, 2, 8, 1500, 128, True, seed=900 + splits, splits=splits, scale=-128 ** -0.5)
    run_case(3, 16, 4, 8, 777, 64, False, seed=910 + splits, splits=splits, scale=-0.2)
