"""ctypes binding of libexattn.so: argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks the
things ctypes cannot (device, dtype, contiguity), allocates the outputs with
``torch.empty`` and calls the C entry point of the same name on torch's current
stream. All arithmetic happens in the HIP kernels; there is no fallback. A
missing library raises an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libexattn.so"

ATTN_BF16 = 0
ATTN_FP16 = 1
FP8_BLOCK = 128

_lib = None


class AttnError(RuntimeError):
    """A non-zero return code of the C ABI."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {attn_strerror(code)} (code {code})")


def library_path() -> str:
    """The in-tree library, or the file named by EXATTN_LIBRARY (another build of it)."""
    return os.environ.get("EXATTN_LIBRARY") or os.path.join(PKG, LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load the in-tree libexattn.so and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -m exact_attention_81_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_tau.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i64p, i64p, i64p, i64p,
                                     f, i, i, vp]
    lib.attn_fwd_strided.restype = i
    lib.attn_fwd_tau.restype = i
    lib.attn_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, vp, i, vp]
    lib.attn_quantize_fp8.restype = i
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, vp,
                                    ctypes.c_size_t, vp]
    lib.attn_fwd_decode.restype = i
    lib.attn_decode_splits.argtypes = [i, i, i, i, i, i, i, i]
    lib.attn_decode_splits.restype = i
    lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i,
                                            vp]
    lib.attn_fwd_decode_noalloc.restype = i
    lib.attn_decode_scratch_bytes.argtypes = []
    lib.attn_decode_scratch_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_bwd.restype = i
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _check(t, name, dtypes, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (BHND)")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, N, d]")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_output(t, name, shape, dtype, device, dense=True):
    """A caller-supplied output: the kernels write every element of ``shape`` through a
    raw pointer, so anything smaller, of another dtype or on another device is refused."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_vector(t, name, numel, dtype, device):
    """A float32 side input read by index (descales): contiguous and at least as long
    as the kernels index it."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _check_strided(t, name, dtypes, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, N, d]")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must be dense along its last dimension")


def _strides(t):
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _fwd(q, k, v, causal, scale, tau, out, lse):
    import torch

    dense = all(t.is_contiguous() for t in (q, k, v)) and (out is None or out.is_contiguous())
    if not dense:
        if tau is not None:
            raise ValueError("attn_fwd_tau takes contiguous tensors")
        return _fwd_strided(q, k, v, causal, scale, out, lse)
    _check(q, "q", (torch.bfloat16, torch.float16))
    _check(k, "k", (q.dtype,), q.device)
    _check(v, "v", (q.dtype,), q.device)
    B, H, n_q, d_qk = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, H, n_kv, d_qk) or v.shape != (B, H, n_kv, d_v):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = d_qk ** -0.5
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=q.dtype, device=q.device)
    _check_output(out, "out", (B, H, n_q, d_v), q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    _check_output(lse, "lse", (B, H, n_q), torch.float32, q.device)
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_FP16
    lib = load_library()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, n_q, n_kv, d_qk, d_v,
            float(scale), int(bool(causal)), dtype]
    if tau is None:
        rc = lib.attn_fwd(*args, _stream(q))
        where = "attn_fwd"
    else:
        rc = lib.attn_fwd_tau(*args, int(tau), _stream(q))
        where = "attn_fwd_tau"
    if rc != 0:
        raise AttnError(rc, where)
    return out, lse


def _fwd_strided(q, k, v, causal, scale, out, lse):
    import torch

    _check_strided(q, "q", (torch.bfloat16, torch.float16))
    _check_strided(k, "k", (q.dtype,), q.device)
    _check_strided(v, "v", (q.dtype,), q.device)
    B, H, n_q, d_qk = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, H, n_kv, d_qk) or v.shape != (B, H, n_kv, d_v):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = d_qk ** -0.5
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=q.dtype, device=q.device)
    _check_strided(out, "out", (q.dtype,))
    _check_output(out, "out", (B, H, n_q, d_v), q.dtype, q.device, dense=False)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    _check_output(lse, "lse", (B, H, n_q), torch.float32, q.device)
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_FP16
    rc = load_library().attn_fwd_strided(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, n_q, n_kv, d_qk, d_v,
        _strides(q), _strides(k), _strides(v), _strides(out), float(scale), int(bool(causal)),
        dtype, _stream(q))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_strided")
    return out, lse


def attn_fwd(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
             out=None, lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O [B,H,N_q,d_v] (dtype of q) and LSE [B,H,N_q] float32.

    Contiguous [B,H,N,d] tensors go to attn_fwd; any other layout whose last dimension
    is dense (e.g. a [B,N,H,d] buffer viewed as [B,H,N,d]) to attn_fwd_strided. ``out``
    may be such a view too.
    """
    return _fwd(q, k, v, causal, scale, None, out, lse)


def attn_fwd_tau(q, k, v, *, tau: int, causal: bool = False, scale: Optional[float] = None,
                 out=None, lse=None):
    """attn_fwd with the rescale threshold tau (0 or 8, in doublings)."""
    return _fwd(q, k, v, causal, scale, tau, out, lse)


def attn_quantize_fp8(x, *, signs=None, transpose: bool = False):
    """e4m3 codes (uint8) and per-128-token float32 descales of a bf16 [B,H,N,d] tensor."""
    import torch

    _check(x, "x", (torch.bfloat16,))
    B, H, N, d = x.shape
    nb = (N + FP8_BLOCK - 1) // FP8_BLOCK
    shape = (B, H, d, N) if transpose else (B, H, N, d)
    x8 = torch.empty(shape, dtype=torch.uint8, device=x.device)
    desc = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    if signs is not None:
        if not signs.is_cuda or signs.dtype != torch.float32 or signs.numel() != d:
            raise ValueError("signs must be a float32 GPU tensor of d elements")
        signs = signs.contiguous()
    rc = load_library().attn_quantize_fp8(_ptr(x), _ptr(x8), _ptr(desc), B, H, N, d, _ptr(signs),
                                          int(bool(transpose)), _stream(x))
    if rc != 0:
        raise AttnError(rc, "attn_quantize_fp8")
    return x8, desc


def attn_fwd_fp8(q8, k8, v8t, q_descale, k_descale, v_descale, *, causal: bool = False,
                 scale: Optional[float] = None, out=None, lse=None):
    """Attention on e4m3 codes; v8t is [B,H,d_v,N_kv]. Returns bf16 O and float32 LSE."""
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v8t", v8t)):
        _check(t, name, (torch.uint8,))
    B, H, n_q, d_qk = q8.shape
    n_kv = k8.shape[2]
    d_v = v8t.shape[2]
    if k8.shape != (B, H, n_kv, d_qk) or v8t.shape != (B, H, d_v, n_kv):
        raise ValueError("shape mismatch between q8, k8 and v8t")
    for name, t in (("k8", k8), ("v8t", v8t)):
        if t.device != q8.device:
            raise ValueError(f"{name} must be on {q8.device}")
    nbq = (n_q + FP8_BLOCK - 1) // FP8_BLOCK
    nbk = (n_kv + FP8_BLOCK - 1) // FP8_BLOCK
    for name, t, nb in (("q_descale", q_descale, nbq), ("k_descale", k_descale, nbk),
                        ("v_descale", v_descale, nbk)):
        _check_vector(t, name, B * H * nb, torch.float32, q8.device)
    if scale is None:
        scale = d_qk ** -0.5
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=torch.bfloat16, device=q8.device)
    _check_output(out, "out", (B, H, n_q, d_v), torch.bfloat16, q8.device)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q8.device)
    _check_output(lse, "lse", (B, H, n_q), torch.float32, q8.device)
    rc = load_library().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8t), _ptr(q_descale),
                                     _ptr(k_descale), _ptr(v_descale), _ptr(out), _ptr(lse),
                                     B, H, n_q, n_kv, d_qk, d_v, float(scale), int(bool(causal)),
                                     _stream(q8))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_fp8")
    return out, lse


def attn_decode_splits(B: int, H: int, H_kv: int, n_q: int, n_kv: int, d: int,
                       num_splits: int = 0) -> int:
    """Key ranges attn_fwd_decode uses on the current device (0 = its own choice)."""
    rc = load_library().attn_decode_splits(B, H, H_kv, n_q, n_kv, d, d, int(num_splits))
    if rc < 0:
        raise AttnError(rc, "attn_decode_splits")
    return rc


def attn_fwd_decode(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                    num_splits: int = 0, out=None, lse=None, workspace=None):
    """Split-KV attention with grouped KV heads: q [B,H,N_q,d], k/v [B,H_kv,N_kv,d].

    Returns O [B,H,N_q,d] (dtype of q) and LSE [B,H,N_q] float32. The workspace for
    the split partials is allocated here (float32 tensor) unless one is passed.
    """
    import torch

    _check(q, "q", (torch.bfloat16, torch.float16))
    _check(k, "k", (q.dtype,), q.device)
    _check(v, "v", (q.dtype,), q.device)
    B, H, n_q, d = q.shape
    H_kv, n_kv = k.shape[1], k.shape[2]
    if k.shape != (B, H_kv, n_kv, d) or v.shape != (B, H_kv, n_kv, v.shape[3]):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    d_v = v.shape[3]
    if scale is None:
        scale = d ** -0.5
    lib = load_library()
    splits = lib.attn_decode_splits(B, H, H_kv, n_q, n_kv, d, d_v, int(num_splits))
    if splits < 0:
        raise AttnError(splits, "attn_fwd_decode")
    need = lib.attn_decode_workspace_bytes(B, H, n_q, d_v, splits)
    if workspace is None and need:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device)
    if workspace is not None and (not workspace.is_cuda or workspace.device != q.device
                                  or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous GPU tensor on {q.device}")
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=q.dtype, device=q.device)
    _check_output(out, "out", (B, H, n_q, d_v), q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    _check_output(lse, "lse", (B, H, n_q), torch.float32, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_FP16
    rc = lib.attn_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, H_kv, n_q, n_kv,
                             d, d_v, float(scale), int(bool(causal)), dtype, int(num_splits),
                             _ptr(workspace), ws_bytes, _stream(q))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_decode")
    return out, lse


def attn_fwd_decode_noalloc(q, k, v, *, out, lse, causal: bool = False,
                            scale: Optional[float] = None, num_splits: int = 0):
    """attn_fwd_decode with the split partials in the library's static scratch: the C
    call allocates nothing, and neither does this binding (``out`` [B,H,N_q,d] and
    ``lse`` [B,H,N_q] float32 are the caller's)."""
    import torch

    _check(q, "q", (torch.bfloat16, torch.float16))
    _check(k, "k", (q.dtype,), q.device)
    _check(v, "v", (q.dtype,), q.device)
    B, H, n_q, d = q.shape
    H_kv, n_kv = k.shape[1], k.shape[2]
    if k.shape != (B, H_kv, n_kv, d) or v.shape != (B, H_kv, n_kv, v.shape[3]):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    d_v = v.shape[3]
    _check_output(out, "out", (B, H, n_q, d_v), q.dtype, q.device)
    _check_output(lse, "lse", (B, H, n_q), torch.float32, q.device)
    if scale is None:
        scale = d ** -0.5
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_FP16
    rc = load_library().attn_fwd_decode_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, H_kv, n_q, n_kv, d, d_v,
        float(scale), int(bool(causal)), dtype, int(num_splits), _stream(q))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_decode_noalloc")
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: Optional[float] = None):
    """dQ, dK, dV (dtype of q) of attn_fwd's output o / lse for the upstream gradient dout."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(t, name, (torch.bfloat16, torch.float16) if name == "q" else (q.dtype,), q.device)
    if not lse.is_cuda or lse.device != q.device or lse.dtype != torch.float32 or \
            not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 GPU tensor on the device of q")
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if k.shape != (B, H, n_kv, d) or v.shape != (B, H, n_kv, d) or o.shape != q.shape or \
            dout.shape != q.shape or lse.shape != (B, H, n_q):
        raise ValueError("shape mismatch between q, k, v, o, dout and lse")
    if scale is None:
        scale = d ** -0.5
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_FP16
    rc = load_library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), B, H, n_q, n_kv, d, d,
                                 float(scale), int(bool(causal)), dtype, _stream(q))
    if rc != 0:
        raise AttnError(rc, "attn_bwd")
    return dq, dk, dv
