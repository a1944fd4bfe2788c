"""Gradients of exact attention (float64): dQ, dK, dV from Q, K, V and dO.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never calls it.

The backward pass of the forward in oracle/attention.py ("FlashAttention 3 and
4: When the Bottleneck Moves", section 3.2, the backward-pass paragraph;
"FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for Asymmetric
Hardware Scaling", Figure 2: five matrix products and two elementwise steps).
Written from the chain rule for one (b, h), with S = scale Q K^T (causal
entries -inf), P = softmax(S) by rows and O = P V:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic
    dS = P * (dP - D)            (elementwise; D broadcast along each row)
    dQ = scale dS K
    dK = scale dS^T Q

A row with no visible key has P = 0 and contributes nothing.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import to_f64


def head_backward(qh, kh, vh, doh, scale: float, causal: bool = False):
    """(dQ, dK, dV, D) for one (batch, head), float64."""
    qh, kh, vh, doh = to_f64(qh), to_f64(kh), to_f64(vh), to_f64(doh)
    n_q, n_kv = qh.shape[0], kh.shape[0]
    s = scale * (qh @ kh.T)
    if causal:
        j = np.arange(n_kv)[None, :]
        limit = np.arange(n_q)[:, None] + (n_kv - n_q)
        s = np.where(j > limit, -np.inf, s)
    m = s.max(axis=1, initial=-np.inf)
    has_key = np.isfinite(m)
    p = np.exp(s - np.where(has_key, m, 0.0)[:, None])
    l = p.sum(axis=1)
    p = np.where(has_key[:, None], p / np.where(has_key, l, 1.0)[:, None], 0.0)
    o = p @ vh
    dv = p.T @ doh
    dp = doh @ vh.T
    d = (doh * o).sum(axis=1)
    ds = p * (dp - d[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv, d


def attention_backward(q, k, v, do, scale: float, causal: bool = False) -> Tuple[np.ndarray, ...]:
    """dQ, dK, dV [B,H,N,d] and D [B,H,N_q] for contiguous BHND inputs, float64."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, H = q.shape[:2]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dd = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], dd[b, h] = head_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv, dd
