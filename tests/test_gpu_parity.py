"""GPU parity of attn_fwd / attn_fwd_tau against the float64 oracle.

Every call goes through the C ABI (ctypes binding). Inputs come from the
seeded generator; the oracle reads the same bfloat16/float16 tensors.
"""
import numpy as np
import pytest
import torch

import exact_attention_81_amd as ea
import oracle
from exact_attention_81_amd import synth
from gpu_util import compare, f64, log, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def run(q, k, v, causal, scale=None, tau=None, out=None, lse=None):
    if tau is None:
        o, l = ea.attn_fwd(q, k, v, causal=causal, scale=scale, out=out, lse=lse)
    else:
        o, l = ea.attn_fwd_tau(q, k, v, tau=tau, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


def check_full(B, H, nq, nkv, dqk, dv, causal, seed, dtype=torch.bfloat16, tau=None):
    label = f"B{B} H{H} Nq{nq} Nkv{nkv} d{dqk}x{dv} causal={causal} {dtype} tau={tau} seed={seed}"
    log("start " + label)
    q, k, v = synth.qkv(B, H, nq, nkv, dqk, dv, seed, dtype)
    scale = dqk ** -0.5
    dq, dk, dv_ = to_dev(q, k, v)
    o, l = run(dq, dk, dv_, causal, scale, tau)
    o_ref, l_ref = oracle.attention(q, k, v, scale, causal)
    return compare(f64(o), f64(l), o_ref, l_ref, label)


# ------------------------------------------------------------------ workloads
def test_tiny_config():
    w = synth.workload("tiny")
    check_full(w.B, w.H, w.N_q, w.N_kv, w.d_qk, w.d_v, w.causal, w.seed)


@pytest.mark.parametrize("causal", [False, True])
def test_single_shape_full(causal):
    w = synth.workload("single", causal=causal)
    log(f"start {w.label()}")
    q, k, v = synth.qkv_for(w)
    dq, dk, dv = to_dev(q, k, v)
    o, l = run(dq, dk, dv, causal, w.scale)
    o_ref, l_ref = oracle.attention_parallel(q, k, v, w.scale, causal)
    compare(f64(o), f64(l), o_ref, l_ref, w.label())


@pytest.mark.parametrize("w", [w for w in synth.workloads() if w.name in ("sweep", "asym")],
                         ids=lambda w: w.label())
def test_large_full(w):
    """Full-size launch (as benchmarked): every element of O and LSE against the oracle."""
    log(f"start {w.label()} (oracle first)")
    q, k, v = synth.qkv_for(w)
    o_ref, l_ref = oracle.attention_parallel(q, k, v, w.scale, w.causal, processes=16)
    dq, dk, dv = to_dev(q, k, v)
    o, l = run(dq, dk, dv, w.causal, w.scale)
    compare(f64(o), f64(l), o_ref, l_ref, w.label())


# ------------------------------------------------------------------ ragged shapes
SHAPES = [
    (1, 1), (17, 17), (127, 129), (129, 127), (255, 257), (257, 255), (300, 300),
    (1, 300), (300, 1), (64, 513), (513, 64), (600, 200),
]


@pytest.mark.parametrize("nq,nkv", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
def test_ragged(nq, nkv, causal, dims):
    check_full(2, 3, nq, nkv, dims[0], dims[1], causal, seed=nq * 7 + nkv + dims[0])


# ------------------------------------------------------------------ many work items
# More (query tile, head) items than the GPU's 256 compute units, in shapes whose
# sequence lengths are whole query tiles: several workgroups run on each compute unit
# in turn, heavy and light causal tiles mixed.
MANY_ITEM_CASES = [
    (3, 88, 256, 256, 128, 128, False),     # 264 items: 8 workgroups take a second one
    (3, 88, 256, 256, 128, 128, True),
    (2, 96, 512, 512, 128, 128, True),      # 384 items, heavy/light causal pairs
    (4, 72, 256, 768, 128, 128, True),      # N_q < N_kv: bottom-right causal alignment
    (4, 72, 256, 768, 64, 64, False),
    (2, 96, 512, 1024, 192, 128, True),
    (4, 64, 512, 512, 64, 64, True),        # 512 items, two rounds
    (2, 64, 1024, 1024, 128, 128, False),   # 512 items
    (1, 128, 1024, 1024, 128, 128, True),   # 512 items, four query tiles per head
    # A workgroup that runs several tiles loads the next tile's first K/V tiles during
    # the current tile's last two iterations: ragged query tiles, N_q > N_kv, key counts
    # just over one and two key tiles, every head dim.
    (2, 80, 300, 300, 128, 128, True),      # 320 items, ragged last query tile
    (2, 80, 300, 200, 128, 128, True),      # N_q > N_kv, first query tile sees 156 keys
    (4, 72, 256, 100, 128, 128, False),     # 288 items of two key tiles each
    (3, 88, 256, 130, 64, 64, False),       # three key tiles, ragged last one
    (3, 88, 256, 320, 192, 128, True),      # d_qk 192
    (5, 64, 512, 512, 128, 128, True),      # 640 items: 2.5 rounds, heavy/light pairs
]


@pytest.mark.parametrize("case", MANY_ITEM_CASES, ids=lambda c: "B{}H{}_{}x{}_d{}x{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "noncausal"))
def test_many_items(case):
    B, H, nq, nkv, dqk, dv, causal = case
    check_full(B, H, nq, nkv, dqk, dv, causal, seed=B * 1000 + H + nq + nkv + dqk)


def test_many_items_fp16():
    check_full(3, 88, 256, 512, 128, 128, True, seed=91, dtype=torch.float16)


@pytest.mark.parametrize("causal", [False, True])
def test_fp16(causal):
    check_full(2, 4, 333, 517, 128, 128, causal, seed=11, dtype=torch.float16)
    check_full(1, 2, 200, 200, 64, 64, causal, seed=12, dtype=torch.float16)


@pytest.mark.parametrize("causal", [False, True])
def test_tau_zero_and_eight_agree(causal):
    q, k, v = synth.qkv(2, 4, 700, 700, 128, 128, seed=21)
    dq, dk, dv = to_dev(q, k, v)
    o_ref, l_ref = oracle.attention(q, k, v, 128 ** -0.5, causal)
    outs = []
    for tau in (0, 8):
        log(f"start tau={tau} causal={causal}")
        o, l = run(dq, dk, dv, causal, tau=tau)
        compare(f64(o), f64(l), o_ref, l_ref, f"tau={tau} causal={causal}")
        outs.append(f64(o))
    assert np.abs(outs[0] - outs[1]).max() <= 2e-2


def test_rescale_exercised_by_growing_scores():
    """Scores that rise along the key axis force many conditional rescales."""
    log("start growing scores")
    q, k, v = synth.qkv(1, 2, 256, 1024, 64, 64, seed=31)
    ramp = torch.linspace(0, 6, 1024).view(1, 1, 1024, 1)
    k = (k.float() + ramp * q.float().mean(dim=2, keepdim=True)).to(torch.bfloat16)
    dq, dk, dv = to_dev(q, k, v)
    for tau in (0, 8):
        o, l = run(dq, dk, dv, False, scale=0.5, tau=tau)
        o_ref, l_ref = oracle.attention(q, k, v, 0.5, False)
        compare(f64(o), f64(l), o_ref, l_ref, f"growing scores tau={tau}")


# ------------------------------------------------------------------ properties
def test_deterministic():
    q, k, v = synth.qkv(2, 8, 1000, 1000, 128, 128, seed=41)
    dq, dk, dv = to_dev(q, k, v)
    log("start determinism")
    a = run(dq, dk, dv, True)
    b = run(dq, dk, dv, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_causal_future_perturbation():
    q, k, v = synth.qkv(1, 2, 512, 512, 128, 128, seed=51)
    dq, dk, dv = to_dev(q, k, v)
    log("start future perturbation")
    o1, l1 = run(dq, dk, dv, True)
    cut = 300
    k2, v2 = dk.clone(), dv.clone()
    k2[:, :, cut + 1:] = torch.randn_like(k2[:, :, cut + 1:].float()).to(k2.dtype) * 4
    v2[:, :, cut + 1:] = torch.randn_like(v2[:, :, cut + 1:].float()).to(v2.dtype) * 4
    o2, l2 = run(dq, k2, v2, True)
    assert torch.equal(o1[:, :, :cut + 1], o2[:, :, :cut + 1])
    assert torch.equal(l1[:, :, :cut + 1], l2[:, :, :cut + 1])
    assert not torch.equal(o1[:, :, cut + 1:], o2[:, :, cut + 1:])


@pytest.mark.parametrize("causal", [False, True])
def test_every_output_written(causal):
    q, k, v = synth.qkv(3, 2, 333, 190, 64, 64, seed=61)
    dq, dk, dv = to_dev(q, k, v)
    out = torch.full((3, 2, 333, 64), float("nan"), dtype=torch.bfloat16, device=dq.device)
    lse = torch.full((3, 2, 333), float("nan"), dtype=torch.float32, device=dq.device)
    log(f"start NaN sentinel causal={causal}")
    o, l = run(dq, dk, dv, causal, out=out, lse=lse)
    assert not torch.isnan(o).any() and not torch.isnan(l).any()
    if causal:  # N_q > N_kv: the first 143 rows see no key
        assert torch.all(o[:, :, :143] == 0) and torch.all(torch.isneginf(l[:, :, :143]))
        assert torch.all(torch.isfinite(l[:, :, 143:]))


def test_closed_forms_on_gpu():
    log("start closed forms")
    q, k, v = synth.qkv(1, 2, 300, 300, 128, 128, seed=71)
    k = k[:, :, :1].expand(-1, -1, 300, -1).contiguous()   # identical keys
    dq, dk, dv = to_dev(q, k, v)
    o, l = run(dq, dk, dv, True)
    vf = v.double()
    mean = torch.cumsum(vf, dim=2) / torch.arange(1, 301, dtype=torch.float64).view(1, 1, 300, 1)
    assert (o.cpu().double() - mean).abs().max().item() <= 1e-2 + 2 ** -8 * mean.abs().max().item()
    # one key: O = v_0 for every query
    q1, k1, v1 = synth.qkv(1, 2, 77, 1, 64, 64, seed=72)
    o1, _ = run(*to_dev(q1, k1, v1), False)
    assert torch.equal(o1.cpu(), v1.expand(-1, -1, 77, -1))
    # scale 0: uniform average
    o0, l0 = run(dq, dk, dv, False, scale=0.0)
    ref = vf.mean(dim=2, keepdim=True).expand(-1, -1, 300, -1)
    assert (o0.cpu().double() - ref).abs().max().item() <= 1e-2
    assert torch.allclose(l0.cpu().double(), torch.full_like(l0.cpu().double(), np.log(300)), atol=1e-4)


def test_scale_argument_and_errors():
    q, k, v = synth.qkv(1, 1, 64, 64, 64, 64, seed=81)
    dq, dk, dv = to_dev(q, k, v)
    log("start scale arg")
    o, l = run(dq, dk, dv, False, scale=0.3)
    o_ref, l_ref = oracle.attention(q, k, v, 0.3, False)
    compare(f64(o), f64(l), o_ref, l_ref, "scale=0.3")
    with pytest.raises(ea.AttnError):
        ea.attn_fwd(dq, dk, dv, scale=float("inf"))
    bad = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device=dq.device)
    with pytest.raises(ea.AttnError):
        ea.attn_fwd(bad, bad, bad)


def test_output_buffers_checked():
    """Caller-supplied O and LSE of the wrong shape, dtype or layout are refused before
    anything is launched."""
    q, k, v = synth.qkv(1, 2, 64, 64, 64, 64, seed=82)
    dq, dk, dv = to_dev(q, k, v)
    log("start output checks")
    dev = dq.device
    for out, lse in ((torch.empty(1, 2, 63, 64, dtype=torch.bfloat16, device=dev), None),
                     (torch.empty(1, 2, 64, 64, dtype=torch.float16, device=dev), None),
                     (None, torch.empty(1, 2, 32, dtype=torch.float32, device=dev)),
                     (None, torch.empty(1, 2, 64, dtype=torch.bfloat16, device=dev)),
                     (None, torch.empty(1, 2, 128, dtype=torch.float32, device=dev)[:, :, ::2])):
        with pytest.raises(ValueError):
            ea.attn_fwd(dq, dk, dv, out=out, lse=lse)
    base = torch.empty(1, 64, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ea.AttnError):  # an O view whose two heads share rows: the C ABI refuses it
        ea.attn_fwd(dq, dk, dv, out=base.unsqueeze(1).expand(1, 2, 64, 64))


# ------------------------------------------------------------------ negative scales
# A negative scale reverses the ordering of the scores. The kernels take the row
# maximum of the scores times |scale| with the sign bits of Q flipped, which is exact.
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale(dims, causal):
    dqk, dv = dims
    q, k, v = synth.qkv(2, 3, 300, 517, dqk, dv, seed=90 + dqk + int(causal))
    dq, dk, dv_ = to_dev(q, k, v)
    for scale in (-dqk ** -0.5, -0.05):
        label = f"negative scale {scale:.4f} d{dqk}x{dv} causal={causal}"
        log("start " + label)
        o, l = run(dq, dk, dv_, causal, scale=scale)
        o_ref, l_ref = oracle.attention(q, k, v, scale, causal)
        compare(f64(o), f64(l), o_ref, l_ref, label)


def test_negative_scale_tau0_fp16_and_many_items():
    q, k, v = synth.qkv(2, 4, 333, 333, 128, 128, seed=95, dtype=torch.float16)
    dq, dk, dv = to_dev(q, k, v)
    o_ref, l_ref = oracle.attention(q, k, v, -0.125, True)
    for tau in (0, 8):
        log(f"start negative scale fp16 tau={tau}")
        o, l = run(dq, dk, dv, True, scale=-0.125, tau=tau)
        compare(f64(o), f64(l), o_ref, l_ref, f"negative scale fp16 tau={tau}")
    q, k, v = synth.qkv(3, 88, 256, 256, 128, 128, seed=96)
    log("start negative scale, 264 items")
    o, l = run(*to_dev(q, k, v), True, scale=-128 ** -0.5)
    o_ref, l_ref = oracle.attention(q, k, v, -128 ** -0.5, True)
    compare(f64(o), f64(l), o_ref, l_ref, "negative scale, 264 items")


# ------------------------------------------------------------------ largest accepted K/V slice
def test_largest_kv_slice_closed_forms():
    """One head whose K and V each hold just over 2^30 elements at d = 128 (the ABI takes
    tensors below 2^31 elements), so the byte count of a head's K or V slice passes 2^31
    (2.15 GB each). The float64 oracle would need 17 GB here, so closed forms decide:
    * K = 0: every score is 0, O is the mean of V and LSE = ln N_kv (bottom-right causal:
      row i averages its first i + N_kv - N_q + 1 values);
    * K's last row = 8 (score 1024 / sqrt(128) against Q = 1, every other score 0): the
      last key outweighs the other 8.4M by e^-90, so O is its value row (3) and LSE is
      its score; under the causal mask only the last query row sees it.
    The split-KV decode path reads the same K and V as one grouped head."""
    dev = require_gpu()
    d, n_q = 128, 64
    n = (1 << 23) + 197  # N_kv * d = 2^30 + 25216 elements; 2^31 + 50432 bytes per tensor
    log(f"start largest K/V slice N_kv={n} d={d}")
    q = torch.ones((1, 1, n_q, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, n, d), dtype=torch.bfloat16, device=dev)
    v = torch.ones((1, 1, n, d), dtype=torch.bfloat16, device=dev)
    v[0, 0, n - 1] = 2.0 ** 20  # exact in bf16
    expect_mean = (n - 1 + 2.0 ** 20) / n
    o, l = run(q, k, v, False)
    compare(f64(o), f64(l), np.full((1, 1, n_q, d), expect_mean), np.full((1, 1, n_q), np.log(n)),
            "K = 0, mean of V")
    od, ld = ea.attn_fwd_decode(q[:, :, :1].expand(1, 8, 1, d).contiguous(), k, v)
    torch.cuda.synchronize()
    compare(f64(od), f64(ld), np.full((1, 8, 1, d), expect_mean), np.full((1, 8, 1), np.log(n)),
            "decode, K = 0, mean of V")

    k[0, 0, n - 1] = 8.0
    v[0, 0, n - 1] = 3.0
    s_star = 8.0 * d / np.sqrt(d)
    lse_star = s_star + np.log1p((n - 1) * np.exp(-s_star))
    o, l = run(q, k, v, False)
    compare(f64(o), f64(l), np.full((1, 1, n_q, d), 3.0), np.full((1, 1, n_q), lse_star),
            "dominant last key")
    o, l = run(q, k, v, True)
    seen = np.arange(n_q) + n - n_q + 1  # keys visible to query row i
    o_ref = np.ones((1, 1, n_q, d))
    o_ref[0, 0, n_q - 1] = 3.0
    l_ref = np.log(seen.astype(np.float64))[None, None, :].copy()
    l_ref[0, 0, n_q - 1] = lse_star
    compare(f64(o), f64(l), o_ref, l_ref, "dominant last key, causal")
