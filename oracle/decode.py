"""Grouped-query attention and the merge of partial results over key splits (float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never calls it.

Grouped KV heads ("Attention at Scale - From FlashAttention to FlashAttention-4",
section "Beyond Training: Attention Kernels for Serving", subsection
"Sequence-Aware Split Heuristic"): H query heads share H_kv key/value heads.
The pages name the scheme (GQA, MQA) but not which query heads share a KV head;
the reading used here is the usual grouping of consecutive heads,

    query head h reads KV head h // (H // H_kv),

so H_kv = H is plain multi-head attention and H_kv = 1 is multi-query attention.

Split keys and the merge (same section, subsection "FlashInfer": attention over
disjoint parts of the key sequence is computed separately and combined by an
associative merge). The pages do not print the operator; it follows from the
softmax definition. For one query row, let part s cover key set K_s with

    LSE_s = ln sum_{j in K_s} exp(S_j),   O_s = sum_{j in K_s} exp(S_j - LSE_s) V_j.

Then over the union of the parts

    LSE = ln sum_s exp(LSE_s),            O = sum_s exp(LSE_s - LSE) O_s.

A part with no visible key has LSE_s = -inf and weight 0; if every part is
empty the row gets O = 0 and LSE = -inf, as in the full definition.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .attention import head, to_f64


def kv_head(h: int, H: int, H_kv: int) -> int:
    """KV head read by query head h (consecutive query heads share one KV head)."""
    return h // (H // H_kv)


def attention_gqa(q, k, v, scale: float, causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """O [B,H,N_q,d_v] and LSE [B,H,N_q] for q [B,H,N_q,d] and k, v [B,H_kv,N_kv,d]."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, n_q, _ = q.shape
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    o = np.empty((B, H, n_q, v.shape[3]))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = head(q[b, h], k[b, g], v[b, g], scale, causal)
    return o, lse


def head_keys(qh, kh, vh, scale: float, causal: bool, lo: int, hi: int):
    """(O, LSE) of one head over the keys [lo, hi) only.

    The causal rule uses absolute key positions: key j is visible to query i iff
    j <= i + (N_kv - N_q), with N_kv the full key count. Same three plain steps as
    the full definition (scores, softmax over the part's keys, times the values).
    """
    qh, kh, vh = to_f64(qh), to_f64(kh), to_f64(vh)
    n_q, n_kv = qh.shape[0], kh.shape[0]
    j = np.arange(lo, hi)
    s = scale * (qh @ kh[lo:hi].T)
    if causal:
        limit = np.arange(n_q)[:, None] + (n_kv - n_q)
        s = np.where(j[None, :] > limit, -np.inf, s)
    m = s.max(axis=1) if hi > lo else np.full(n_q, -np.inf)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (p @ vh[lo:hi]) / l[:, None]
        lse = m_safe + np.log(l)
    o = np.where(has_key[:, None], o, 0.0)
    lse = np.where(has_key, lse, -np.inf)
    return o, lse


def merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Combine partial (O_s, LSE_s) over disjoint key sets into (O, LSE).

    o_parts[s] has shape [..., d_v], lse_parts[s] the matching [...].
    """
    o_parts = [to_f64(o) for o in o_parts]
    lse_parts = [to_f64(x) for x in lse_parts]
    m = np.max(np.stack(lse_parts), axis=0)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    w = [np.exp(x - m_safe) for x in lse_parts]          # exp(-inf) = 0 for empty parts
    total = sum(w)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = sum(wi[..., None] * oi for wi, oi in zip(w, o_parts)) / total[..., None]
        lse = m_safe + np.log(total)
    o = np.where(has_key[..., None], o, 0.0)
    lse = np.where(has_key, lse, -np.inf)
    return o, lse
