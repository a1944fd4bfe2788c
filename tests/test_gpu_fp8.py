"""GPU parity of the fp8 path: the quantiser bit-exact against the oracle's
codec, and the fp8 attention forward against the float64 oracle."""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import log, to_dev

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
