"""The seeded input generator: deterministic, right shapes, right recipe."""
import torch

from exact_attention_81_amd import synth


def test_workload_table():
    ws = synth.workloads()
    assert len(ws) == 1 + 2 + 12 + 1 + 1
    for w in ws:
        if w.name == "sweep":
            assert w.B * w.N_q == 16384 and w.H == 16 and w.d_qk == 128
    w = synth.workload("asym")
    assert (w.d_qk, w.d_v, w.causal, w.N_q) == (192, 128, True, 8192)
    assert abs(w.scale - 192 ** -0.5) < 1e-15
    w2 = synth.workload("single", causal=False)
    assert w2.flops() == 4 * 4 * 16 * 2048 ** 2 * 128
    assert synth.workload("single", causal=True).flops() == w2.flops() / 2


def test_qkv_deterministic_and_ordered():
    a = synth.qkv(1, 2, 5, 7, 8, 4, seed=3)
    b = synth.qkv(1, 2, 5, 7, 8, 4, seed=3)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    g = torch.Generator().manual_seed(3)
    q = torch.randn((1, 2, 5, 8), generator=g).to(torch.bfloat16)
    assert torch.equal(q, a[0])
    assert a[1].shape == (1, 2, 7, 8) and a[2].shape == (1, 2, 7, 4)


def test_fp8_inputs_outliers():
    s, q, k, v = synth.fp8_inputs(1, 2, 256, 128, seed=5)
    assert set(s.tolist()) <= {-1.0, 1.0} and s.shape == (128,)
    frac = (q.float().abs() > 6).float().mean().item()
    assert 0.002 < frac < 0.008
    s0, q0, _, _ = synth.fp8_inputs(1, 2, 256, 128, seed=5, outlier_frac=0.0)
    assert torch.equal(s0, s) and q0.float().abs().max() < 7
