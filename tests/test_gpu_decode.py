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


def _decode_ws_bytes(B, H, nq, d, splits):
    return ea.load_library().attn_decode_workspace_bytes(B, H, nq, d, splits)


def test_decode_workspace_leftover_bytes_and_reuse():
    """Whatever bytes the split workspace holds on entry (zeros, all ones, random bytes,
    another call's partials) the result is the same, bit for bit, and calls that reuse
    one workspace, also with other shapes, agree with fresh ones."""
    B, H, H_kv, nq, nkv, d = 2, 16, 4, 3, 2100, 128
    q, k, v = synth.qkv_gqa(B, H, H_kv, nq, nkv, d, seed=941)
    dq, dk, dv = to_dev(q, k, v)
    splits = ea.attn_decode_splits(B, H, H_kv, nq, nkv, d, 6)
    assert splits == 6
    need = _decode_ws_bytes(B, H, nq, d, splits)
    nwords = (need + 3) // 4
    log(f"start decode workspace fills B{B} H{H} Hkv{H_kv} Nq{nq} Nkv{nkv} splits={splits}")
    ref_o, ref_l = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_gqa(q, k, v, d ** -0.5, True)
    compare(f64(ref_o), f64(ref_l), o_ref, lse_ref, "decode reference call")
    gen = torch.Generator().manual_seed(942)
    fills = {
        "zeros": torch.zeros(nwords, dtype=torch.int32),
        "ones": torch.full((nwords,), -1, dtype=torch.int32),
        "random": torch.randint(-2 ** 31, 2 ** 31 - 1, (nwords,), dtype=torch.int32, generator=gen),
    }
    for name, fill in fills.items():
        ws = fill.to(dq.device).view(torch.float32)
        for rep in range(3):   # the same workspace again: its counters carry over
            o, l = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o, ref_o) and torch.equal(l, ref_l), (name, rep)
    # another shape through the same workspace, then the first again
    q2, k2, v2 = synth.qkv_gqa(1, 8, 8, 1, 3000, 128, seed=943)
    d2q, d2k, d2v = to_dev(q2, k2, v2)
    s2 = ea.attn_decode_splits(1, 8, 8, 1, 3000, 128, 11)
    assert _decode_ws_bytes(1, 8, 1, 128, s2) <= need
    o2, l2 = ea.attn_fwd_decode(d2q, d2k, d2v, num_splits=11, workspace=ws)
    o, l = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    o2_ref, l2_ref = oracle.attention_gqa(q2, k2, v2, 128 ** -0.5, False)
    compare(f64(o2), f64(l2), o2_ref, l2_ref, "decode second shape, shared workspace")
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_decode_graph_replays():
    """attn_fwd_decode (split kernel and merge kernel) captured in a HIP graph: every
    replay, on new inputs copied into the captured buffers, is checked against an eager
    call on the same inputs, with eager work and synchronisations between the replays.
    The call issues no memset."""
    B, H, H_kv, nq, nkv, d = 2, 8, 2, 2, 2500, 128
    splits = 5
    dev = torch.device("cuda:0")
    q0, k0, v0 = synth.qkv_gqa(B, H, H_kv, nq, nkv, d, seed=951)
    dq, dk, dv = to_dev(q0, k0, v0)
    out = torch.empty((B, H, nq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    ws = torch.empty(((_decode_ws_bytes(B, H, nq, d, splits) + 3) // 4,), dtype=torch.float32,
                     device=dev)
    log("start decode graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream, as torch asks
        ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        qn, kn, vn = synth.qkv_gqa(B, H, H_kv, nq, nkv, d, seed=952 + rep)
        dq.copy_(qn.to(dev)); dk.copy_(kn.to(dev)); dv.copy_(vn.to(dev))
        torch.cuda.synchronize()
        log(f"decode graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        e_o, e_l = ea.attn_fwd_decode(dq, dk, dv, causal=True, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, e_o) and torch.equal(lse, e_l), rep
        if rep == 0:
            o_ref, lse_ref = oracle.attention_gqa(qn, kn, vn, d ** -0.5, True)
            compare(f64(out), f64(lse), o_ref, lse_ref, "decode graph replay 0")
