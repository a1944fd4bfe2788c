"""fp8 e4m3 codec, random-sign Hadamard rotation and per-block quantisation.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never calls it.

Sources:
  * "FlashAttention 3 and 4: When the Bottleneck Moves", section 2.2: eight-bit
    tensor-core arithmetic at about twice the 16-bit rate; every block of values
    gets its own scale; Q and K are multiplied by one fixed random rotation R
    before quantising, which cancels in the scores because R R^T = I.
  * "Attention at Scale - From FlashAttention to FlashAttention-4", section
    "The Evolution" (FlashAttention-3): FP8 with block quantisation.

Readings where the pages are silent (each listed in the design notes):
  * The 8-bit format is OCP e4m3 ("e4m3fn"): 1 sign, 4 exponent (bias 7) and
    3 mantissa bits, subnormals, no infinities, the all-ones pattern is NaN, and
    the largest finite magnitude is 448. Rounding is to nearest, ties to even,
    and magnitudes beyond 448 saturate to 448.
  * The rotation is R = diag(sigma) H_d / sqrt(d), sigma a seeded +-1 vector and
    H_d the Sylvester Hadamard matrix. Only Q and K are rotated.
  * A block is 128 consecutive tokens of one (batch, head) by all d coordinates.
    Its scale is s = amax / 448 (amax of the rotated block), so the largest
    element maps to +-448. An all-zero block gets codes 0 and scale 0.
  * Codes are computed from the unnormalised rotation y = x diag(sigma) H_d,
    which is exact in float64 for bfloat16 inputs, as
        code = e4m3(float32(y * (448 / amax)))
    with the product and the quotient rounded in float64 and the float32 step
    rounding to nearest even. 1/sqrt(d) cancels between y and amax, so it only
    enters the stored descale: float32(amax / (448 * sqrt(d))) when rotated,
    float32(amax / 448) otherwise. Dequantised values code * descale then
    approximate x R (rotated) or x (not rotated).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import to_f64

E4M3_MAX = 448.0
E4M3_NAN = 0x7F
BLOCK_TOKENS = 128


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each e4m3 byte (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Round each value to e4m3: nearest, ties to even, saturating at +-448.

    The input is taken as given (float32 inputs are exact in float64); the one
    rounding happens here.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.abs(np.where(nan, 0.0, x))
    neg = np.signbit(x) & ~nan
    # Binade of |x|: a = f * 2**E with f in [0.5, 1), so floor(log2 a) = E - 1.
    _, E = np.frexp(a)
    e = np.maximum(E - 1, -6)                    # below 2**-6: subnormal spacing
    quantum = np.exp2((e - 3).astype(np.float64))  # 3 mantissa bits
    n = np.rint(a / quantum)                     # exact division; rint ties to even
    val = np.minimum(n * quantum, E4M3_MAX)      # saturate
    # Encode the rounded magnitude.
    _, E2 = np.frexp(val)
    e2 = E2 - 1
    is_sub = val < 2.0 ** -6
    mant_sub = np.rint(val / 2.0 ** -9).astype(np.int64)          # 0..7
    biased = np.clip(e2 + 7, 1, 15)
    mant_norm = np.rint((val / np.exp2(e2.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    code = np.where(is_sub, mant_sub, (biased << 3) | np.clip(mant_norm, 0, 7))
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs) -> np.ndarray:
    """R = diag(signs) H_d / sqrt(d), an orthogonal d x d matrix."""
    s = to_f64(signs).reshape(-1)
    d = s.shape[0]
    return (s[:, None] * hadamard(d)) / np.sqrt(d)


def quantize_blocks(x, signs=None, block: int = BLOCK_TOKENS) -> Tuple[np.ndarray, np.ndarray]:
    """Per-block e4m3 quantisation of x [B,H,N,d], rotated when ``signs`` is given.

    Returns codes uint8 [B,H,N,d] and descale float32 [B,H,ceil(N/block)].
    """
    x = to_f64(x)
    B, H, N, d = x.shape
    if signs is not None:
        s = to_f64(signs).reshape(-1)
        y = x @ (s[:, None] * hadamard(d))   # exact: sums of +-bfloat16 values
    else:
        y = x
    nb = (N + block - 1) // block
    codes = np.empty((B, H, N, d), dtype=np.uint8)
    descale = np.empty((B, H, nb), dtype=np.float32)
    div = 448.0 * np.sqrt(float(d)) if signs is not None else 448.0
    for i in range(nb):
        yb = y[:, :, i * block:(i + 1) * block, :]
        amax = np.abs(yb).max(axis=(2, 3))                  # [B,H]
        zero = amax == 0.0
        with np.errstate(divide="ignore"):
            ratio = np.where(zero, 0.0, E4M3_MAX / np.where(zero, 1.0, amax))
        scaled = (yb * ratio[:, :, None, None]).astype(np.float32)
        codes[:, :, i * block:(i + 1) * block, :] = e4m3_encode(scaled)
        descale[:, :, i] = (amax / div).astype(np.float32)
    return codes, descale


def dequantize_blocks(codes, descale, block: int = BLOCK_TOKENS) -> np.ndarray:
    """float64 code * descale, the tensor the fp8 attention actually consumes."""
    vals = e4m3_decode(codes)
    N = vals.shape[2]
    sc = np.repeat(np.asarray(descale, dtype=np.float64), block, axis=2)[:, :, :N]
    return vals * sc[..., None]
