"""Fused exact-attention forward for AMD MI355X (gfx950).

The compute path is a HIP library, ``libexattn.so``, behind a C ABI
(``include/exattn.h``). This package holds its sources (``csrc/``), the build
step and a thin ctypes binding with the same entry-point names. Importing the
package does not load the library; the first call does, and fails loudly when
the library has not been built.
"""
from .binding import (  # noqa: F401
    AttnError,
    attn_bwd,
    attn_decode_splits,
    attn_fwd,
    attn_fwd_decode,
    attn_fwd_decode_noalloc,
    attn_fwd_fp8,
    attn_fwd_tau,
    attn_quantize_fp8,
    attn_strerror,
    library_path,
    load_library,
)
