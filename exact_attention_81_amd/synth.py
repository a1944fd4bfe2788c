"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random tensors. It holds none of the attention
arithmetic, so both the CPU oracle side of the tests and the HIP path can take
their inputs from it without sharing any of the method's code.

Recipe (the same everywhere: tests, smoke check, benchmark):
  * ``torch.Generator('cpu').manual_seed(seed)``;
  * ``torch.randn`` in float32, then rounded to bfloat16 (round-to-nearest-even)
    or float16;
  * draw order Q, K, V;
  * for the fp8 workload the 128 rotation signs are drawn first, then for each
    of Q, K, V its normals followed by its outlier mask (i.i.d. Bernoulli with
    probability ``outlier_frac``); masked coordinates are multiplied by
    ``outlier_mult`` before the rounding to bfloat16.

The outlier construction follows the observation, in "FlashAttention 3 and 4:
When the Bottleneck Moves" section 2.2, that transformer activations sit mostly
near zero with a few large outliers.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-forward problem shape."""

    name: str
    B: int
    H: int
    N_q: int
    N_kv: int
    d_qk: int
    d_v: int
    causal: bool
    seed: int
    fp8: bool = False

    @property
    def scale(self) -> float:
        return float(self.d_qk) ** -0.5

    def flops(self) -> float:
        """Algorithmic flops: 2*B*H*N_q*N_kv*(d_qk+d_v), halved when causal."""
        f = 2.0 * self.B * self.H * self.N_q * self.N_kv * (self.d_qk + self.d_v)
        return f * 0.5 if self.causal else f

    def label(self) -> str:
        c = "causal" if self.causal else "noncausal"
        dt = "fp8" if self.fp8 else "bf16"
        return (f"{self.name}:B{self.B}_H{self.H}_Nq{self.N_q}_Nkv{self.N_kv}"
                f"_d{self.d_qk}x{self.d_v}_{c}_{dt}")


def seed_for(config: int, index: int = 0) -> int:
    return 1000 + 10 * config + index


SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)


def workloads() -> List[Workload]:
    """The five workload families, each causal variant listed separately."""
    out: List[Workload] = []
    out.append(Workload("tiny", 1, 2, 256, 256, 64, 64, False, seed_for(1)))
    for c in (False, True):
        out.append(Workload("single", 4, 16, 2048, 2048, 128, 128, c, seed_for(2)))
    for i, n in enumerate(SWEEP_N):
        for c in (False, True):
            out.append(Workload("sweep", 16384 // n, 16, n, n, 128, 128, c, seed_for(3, i)))
    out.append(Workload("asym", 1, 16, 8192, 8192, 192, 128, True, seed_for(4)))
    out.append(Workload("fp8", 4, 16, 4096, 4096, 128, 128, False, seed_for(5), fp8=True))
    return out


def workload(name: str, causal: Optional[bool] = None, N: Optional[int] = None) -> Workload:
    for w in workloads():
        if w.name != name:
            continue
        if causal is not None and w.causal != causal:
            continue
        if N is not None and w.N_q != N:
            continue
        return w
    raise KeyError(f"no workload {name} causal={causal} N={N}")


def qkv(B: int, H: int, N_q: int, N_kv: int, d_qk: int, d_v: int, seed: int,
        dtype: torch.dtype = torch.bfloat16):
    """Q [B,H,N_q,d_qk], K [B,H,N_kv,d_qk], V [B,H,N_kv,d_v] ~ N(0,1), CPU tensors."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, H, N_q, d_qk), generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn((B, H, N_kv, d_qk), generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn((B, H, N_kv, d_v), generator=g, dtype=torch.float32).to(dtype)
    return q, k, v


def qkv_gqa(B: int, H: int, H_kv: int, N_q: int, N_kv: int, d: int, seed: int,
            dtype: torch.dtype = torch.bfloat16):
    """Q [B,H,N_q,d], K and V [B,H_kv,N_kv,d] ~ N(0,1) (grouped KV heads), CPU tensors."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, H, N_q, d), generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn((B, H_kv, N_kv, d), generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn((B, H_kv, N_kv, d), generator=g, dtype=torch.float32).to(dtype)
    return q, k, v


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """A decode-shaped problem: few queries per head, grouped KV heads, long keys."""

    name: str
    B: int
    H: int
    H_kv: int
    N_q: int
    N_kv: int
    d: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return float(self.d) ** -0.5

    def hbm_bytes(self) -> int:
        """Algorithmic HBM traffic of one call: K and V read once, Q read, O and LSE written."""
        kv = 2 * self.B * self.H_kv * self.N_kv * self.d * 2
        qo = 2 * self.B * self.H * self.N_q * self.d * 2
        return kv + qo + 4 * self.B * self.H * self.N_q

    def label(self) -> str:
        c = "causal" if self.causal else "noncausal"
        return (f"{self.name}:B{self.B}_H{self.H}_Hkv{self.H_kv}_Nq{self.N_q}_Nkv{self.N_kv}"
                f"_d{self.d}_{c}_bf16")


def decode_workload() -> DecodeWorkload:
    """Single-token decode over a 16k-token cache with 8-way grouped KV heads."""
    return DecodeWorkload("decode", 8, 64, 8, 1, 16384, 128, False, seed_for(6))


def qkv_for(w: Workload, dtype: torch.dtype = torch.bfloat16):
    return qkv(w.B, w.H, w.N_q, w.N_kv, w.d_qk, w.d_v, w.seed, dtype)


def fp8_inputs(B: int, H: int, N: int, d: int, seed: int, outlier_frac: float = 0.005,
               outlier_mult: float = 30.0):
    """Signs [d] (+-1, float32), then Q, K, V [B,H,N,d] bfloat16 with outliers.

    With ``outlier_frac == 0`` the mask is still drawn (so the normals are the
    same draws) but nothing is scaled.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    signs = torch.randint(0, 2, (d,), generator=g, dtype=torch.int64).to(torch.float32) * 2 - 1
    out = []
    for _ in range(3):
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        mask = torch.rand((B, H, N, d), generator=g, dtype=torch.float32) < outlier_frac
        x = torch.where(mask, x * outlier_mult, x)
        out.append(x.to(torch.bfloat16))
    return signs, out[0], out[1], out[2]
