"""attn_fwd_decode_noalloc (the decode entry point that allocates nothing) against
attn_fwd_decode with a caller workspace, through the C ABI.

Both run the same kernels with the same split count; only where the split partials
live differs (the library's static device scratch, or the caller's buffer), so the
outputs must be bit-identical, and both must meet the oracle gate. Two calls in a row,
the second smaller than the first, check that nothing the first call left in the
scratch leaks into the second. The binding allocates nothing either: the caching
allocator's count of allocated bytes is unchanged across the calls.
"""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import compare, f64, log, require_gpu

pytestmark = pytest.mark.gpu

# (B, H, H_kv, N_q, N_kv, d, causal): the decode workload, then a smaller problem
CALLS = [(8, 64, 8, 1, 16384, 128, False), (2, 16, 2, 8, 1500, 128, True)]


def test_noalloc_matches_workspace_entry():
    dev = require_gpu()
    for B, H, H_kv, nq, nkv, d, causal in CALLS:
        label = f"noalloc decode B{B} H{H} Hkv{H_kv} Nq{nq} Nkv{nkv} d{d} causal={causal}"
        log("start " + label)
        q, k, v = synth.qkv_gqa(B, H, H_kv, nq, nkv, d, seed=B * 100 + nkv)
        dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
        splits = ea.attn_decode_splits(B, H, H_kv, nq, nkv, d)
        assert splits > 1, "the case must use the split partials"
        need = ea.load_library().attn_decode_workspace_bytes(B, H, nq, d, splits)
        assert need <= ea.load_library().attn_decode_scratch_bytes()
        o_ws, l_ws = ea.attn_fwd_decode(dq, dk, dv, causal=causal)
        o_na = torch.full_like(o_ws, float("nan"))
        l_na = torch.full_like(l_ws, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        ea.attn_fwd_decode_noalloc(dq, dk, dv, out=o_na, lse=l_na, causal=causal)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(dev) == before
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), label
        o_ref, l_ref = oracle.attention_gqa(q, k, v, d ** -0.5, causal)
        compare(f64(o_na), f64(l_na), o_ref, l_ref, label)


def test_noalloc_refuses_oversized_split_partials():
    dev = require_gpu()
    q, k, v = synth.qkv_gqa(8, 64, 8, 1, 16384, 128, seed=5)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((8, 64, 1, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((8, 64, 1), dtype=torch.float32, device=dev)
    log("start noalloc oversized")
    with pytest.raises(ea.AttnError) as err:
        ea.attn_fwd_decode_noalloc(dq, dk, dv, out=out, lse=lse, num_splits=256)
    assert err.value.code == -9
