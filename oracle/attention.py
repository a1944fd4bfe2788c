"""Naive float64 attention: the exact result the fused forward must reproduce.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never calls it.

What is computed (for every batch b and head h, inputs converted exactly from
their stored dtype to float64):

    S    = scale * Q K^T                       (N_q x N_kv, fully materialised)
    S_ij = -inf  if causal and j > i + (N_kv - N_q)
    m_i  = max_j S_ij ;  P_ij = exp(S_ij - m_i) ;  l_i = sum_j P_ij
    O_i  = (sum_j P_ij V_j) / l_i ;  LSE_i = m_i + ln l_i
    rows with no visible key: O_i = 0, LSE_i = -inf

The three steps (score matrix, softmax, multiply by the values) are the naive
algorithm of "Attention at Scale - From FlashAttention to FlashAttention-4",
section "The Problem". That page's section "The Evolution" (FlashAttention)
and "FlashAttention 3 and 4: When the Bottleneck Moves" section 4 state that
the tiled, online-softmax method computes exactly this; section 3.2 of the
latter explains that the conditionally rescaled variant divides, once at the
end, by the exact row maximum and the exact softmax denominator, which are the
m_i and l_i above.

Readings where the pages are silent (each listed in the design notes):
  * LSE is the natural-log logsumexp of the scaled scores.
  * Causal masking is aligned bottom-right: key j is visible to query i iff
    j <= i + (N_kv - N_q); this is the lower-triangular mask when N_q == N_kv.
  * A row with no visible key returns O = 0 and LSE = -inf (log of an empty sum).

Large problems are processed in chunks of full rows; each chunk still holds the
complete score rows, so the softmax stays the plain two-pass one.
"""
from __future__ import annotations

import os
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def to_f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor (any float dtype) or array to float64."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _head_rows(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float,
               causal: bool, rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """O and LSE for the query rows ``rows`` of one (batch, head)."""
    n_q = qh.shape[0]
    n_kv = kh.shape[0]
    # Step 1: the score rows, S = scale * q_i . k_j for every key j.
    s = scale * (qh[rows] @ kh.T)
    if causal:
        j = np.arange(n_kv)[None, :]
        limit = rows[:, None] + (n_kv - n_q)
        s = np.where(j > limit, -np.inf, s)
    # Step 2: softmax over each full row (two passes: max, then exp and sum).
    m = s.max(axis=1) if n_kv > 0 else np.full(len(rows), -np.inf)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    p = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1)
    # Step 3: multiply by the values and normalise by the denominator.
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (p @ vh) / l[:, None]
        lse = m_safe + np.log(l)
    o = np.where(has_key[:, None], o, 0.0)
    lse = np.where(has_key, lse, -np.inf)
    return o, lse


def head(qh, kh, vh, scale: float, causal: bool = False,
         rows: Optional[Sequence[int]] = None,
         max_bytes: int = 1 << 28) -> Tuple[np.ndarray, np.ndarray]:
    """O [len(rows), d_v] and LSE [len(rows)] for one (batch, head), float64."""
    qh, kh, vh = to_f64(qh), to_f64(kh), to_f64(vh)
    n_q, n_kv = qh.shape[0], kh.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    chunk = max(1, int(max_bytes // (8 * max(n_kv, 1))))
    o = np.empty((len(rows), vh.shape[1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        o[a:a + chunk], lse[a:a + chunk] = _head_rows(qh, kh, vh, scale, causal, r)
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """O [B,H,N_q,d_v] and LSE [B,H,N_q] in float64 for contiguous BHND inputs."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, n_q, _ = q.shape
    o = np.empty((B, H, n_q, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def attention_rows(q, k, v, scale: float, causal: bool,
                   picks: Iterable[Tuple[int, int, int]]) -> Tuple[np.ndarray, np.ndarray]:
    """O and LSE of selected outputs, one (b, h, query row) triple at a time.

    Every row still sees its full key sequence, so this is the same definition
    evaluated on a sample of the outputs of a problem too large to run whole.
    """
    picks = list(picks)
    o = []
    lse = []
    for b, h, i in picks:
        oh, lh = head(q[b, h], k[b, h], v[b, h], scale, causal, rows=[i])
        o.append(oh[0])
        lse.append(lh[0])
    return np.array(o), np.array(lse)


# ----------------------------------------------------------------------------
# Parallel driver: one (b, h) per task, BLAS single-threaded per worker.
# ----------------------------------------------------------------------------
_SHARED = {}


def _worker_init(q, k, v, scale, causal):
    try:
        from threadpoolctl import threadpool_limits

        _SHARED["limit"] = threadpool_limits(1)
    except ImportError:  # pragma: no cover - threadpoolctl is installed here
        pass
    _SHARED.update(q=q, k=k, v=v, scale=scale, causal=causal)


def _worker_head(bh):
    b, h = bh
    s = _SHARED
    return bh, head(s["q"][b, h], s["k"][b, h], s["v"][b, h], s["scale"], s["causal"])


def attention_parallel(q, k, v, scale: float, causal: bool = False,
                       processes: Optional[int] = None,
                       heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Same result as ``attention`` (for the listed heads), over a fork pool.

    Returns (o, lse) indexed like ``heads`` when given, else full tensors.
    Workers are forked, so call this before the GPU is touched.
    """
    import multiprocessing as mp

    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H = q.shape[:2]
    todo = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    processes = processes or min(16, os.cpu_count() or 1)
    ctx = mp.get_context("fork")
    with ctx.Pool(processes, initializer=_worker_init,
                  initargs=(q, k, v, scale, causal)) as pool:
        res = dict(pool.map(_worker_head, todo))
    if heads is not None:
        return [res[bh] for bh in todo]
    o = np.empty((B, H, q.shape[2], v.shape[3]))
    lse = np.empty((B, H, q.shape[2]))
    for (b, h), (oh, lh) in res.items():
        o[b, h], lse[b, h] = oh, lh
    return o, lse
