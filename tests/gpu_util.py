"""Helpers for the GPU parity tests: device placement, gates, case logging."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest

# Tolerances on O (bfloat16 / float16 output) and LSE, against the float64 oracle.
#   * max abs 1e-2 and mean abs 1e-3 on O, LSE within 1e-3 are the stated gates;
#   * the output itself is rounded to 16 bits, whose half unit in the last place
#     is up to 2^-8 |O| (bfloat16; the "Ideal FP64 -> BF16" row of Table 2 of the
#     FlashAttention-4 paper puts the worst relative rounding error at 3.89e-3),
#     so the per-element bound is 1e-2 + 2^-8 |O_ref|. The raw max abs is
#     reported next to 1e-2.
O_ATOL = 1e-2
O_RTOL = 2.0 ** -8
O_MEAN = 1e-3
LSE_ATOL = 1e-3


def log(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a GPU (select with -m 'not gpu' on CPU hosts)")
    return torch.device("cuda:0")


def to_dev(*ts):
    dev = require_gpu()
    return [t.to(dev) for t in ts]


def f64(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def record(label: str, stats: dict) -> None:
    """Append one case's error figures as a JSON line to the file named by
    EXATTN_PARITY_RECORD (nothing when it is unset)."""
    path = os.environ.get("EXATTN_PARITY_RECORD")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(dict(case=label, **stats)) + "\n")


def compare(o_gpu, lse_gpu, o_ref, lse_ref, label: str, atol=O_ATOL, rtol=O_RTOL,
            mean_tol=O_MEAN, lse_tol=LSE_ATOL):
    """Gate GPU outputs (numpy float64) against the oracle; returns the stats."""
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite O"
    err = np.abs(o_gpu - o_ref)
    bound = atol + rtol * np.abs(o_ref)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 worst_ratio=float((err / bound).max()))
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{label}: LSE finiteness differs"
    assert np.all(lse_gpu[~fin] == lse_ref[~fin]), f"{label}: empty rows must have LSE -inf"
    stats["lse_max_abs"] = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    stats["elements"] = int(err.size)
    # The part of the error no 16-bit output can avoid: the exact result rounded to
    # bfloat16 (reported when every GPU value is a bfloat16 value).
    import torch

    og = torch.from_numpy(np.ascontiguousarray(o_gpu))
    if torch.equal(og.to(torch.bfloat16).double(), og):
        ideal = np.abs(torch.from_numpy(np.ascontiguousarray(o_ref)).to(torch.bfloat16).double().numpy()
                       - o_ref)
        stats["bf16_rounding_max_abs"] = float(ideal.max())
        stats["max_abs_beyond_rounding"] = float((err - ideal).max())
    log(f"{label}: O max abs {stats['max_abs']:.3e} (vs 1e-2), mean abs {stats['mean_abs']:.3e}, "
        f"worst err/bound {stats['worst_ratio']:.3f}, LSE max abs {stats['lse_max_abs']:.3e}, "
        f"exact result rounded to bf16: max abs {stats.get('bf16_rounding_max_abs', float('nan')):.3e}")
    record(label, stats)
    assert stats["worst_ratio"] <= 1.0, f"{label}: elementwise O gate failed {stats}"
    assert stats["mean_abs"] <= mean_tol, f"{label}: mean abs gate failed {stats}"
    assert stats["lse_max_abs"] <= lse_tol, f"{label}: LSE gate failed {stats}"
    return stats
