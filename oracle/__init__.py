"""CPU oracle for the fused exact-attention forward (float64, plain numpy).

TEST INFRASTRUCTURE. Only ``tests/``, the smoke check and the benchmark's CPU
baseline leg may import this package. It shares no code with the HIP path and
imports nothing from it; the two meet only on inputs drawn by the seeded
generators.
"""
from .attention import attention, attention_parallel, attention_rows, head, to_f64  # noqa: F401
from .fp8 import (  # noqa: F401
    BLOCK_TOKENS,
    E4M3_MAX,
    dequantize_blocks,
    e4m3_decode,
    e4m3_encode,
    hadamard,
    quantize_blocks,
    rotation,
)
from .decode import attention_gqa, head_keys, kv_head, merge  # noqa: F401
from .backward import attention_backward, head_backward  # noqa: F401
