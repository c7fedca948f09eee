"""QK-Norm on MI355X (gfx950): Python binding of the C-ABI library.

This module only marshals arguments: torch tensors supply device pointers and
the current HIP stream, and every step of the computation runs in the HIP
kernels of ``libqknorm.so``.  There is no CPU fallback -- if the library is
not built, or a tensor is not on the GPU, the call raises.

The four entry points keep the C names and semantics (``include/qknorm.h``):

    qknorm_per_head(qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps)
    qknorm_layerwise(qkv, wq, wk, gamma_q, gamma_k, eps, nshards)
    qknorm_partial_sumsq(qkv, wq, wk, nshards, part_q, part_k)
    qknorm_apply_scalar(qkv, wq, wk, part_q, part_k, norm_wq, norm_wk, gamma_q, gamma_k, eps)

``qkv`` is float32, bfloat16 or float16 with gamma of the same dtype, or
float8_e4m3fn with bfloat16 gamma.  It is a [T, ...] tensor whose rows are
contiguous within themselves
(``stride(-1) == 1`` and each row packed); its row pitch is ``stride(0)``.
All calls normalise in place and are enqueued on ``stream`` (default: torch's
current stream).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqknorm.so")

QKNORM_F32 = 0
QKNORM_BF16 = 1
QKNORM_F16 = 2
QKNORM_FP8_E4M3 = 3
QKNORM_OK = 0
QKNORM_E_NULLPTR = -1
QKNORM_E_SHAPE = -2
QKNORM_E_ALIGN = -3
QKNORM_E_DTYPE = -4
QKNORM_E_UNSUPPORTED = -5
QKNORM_E_EPS = -6
QKNORM_E_HIP = -7

EXPORTED = ("qknorm_per_head", "qknorm_layerwise", "qknorm_partial_sumsq",
            "qknorm_apply_scalar", "qknorm_strerror", "qknorm_abi_version")

_lib = None


class QKNormError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} (code {code})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"QK-Norm HIP library not built: {path} is missing "
                           "(run `python -m qk_norm_amd.build` or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.qknorm_per_head.argtypes = [P, I64, I64, I32, I32, I32, P, P, F, I32, P]
    lib.qknorm_layerwise.argtypes = [P, I64, I64, I64, I64, P, P, F, I32, I32, P]
    lib.qknorm_partial_sumsq.argtypes = [P, I64, I64, I64, I64, I32, P, P, I32, P]
    lib.qknorm_apply_scalar.argtypes = [P, I64, I64, I64, I64, P, P, I32, I64, I64, P, P, F, I32, P]
    for name in ("qknorm_per_head", "qknorm_layerwise", "qknorm_partial_sumsq",
                 "qknorm_apply_scalar", "qknorm_abi_version"):
        getattr(lib, name).restype = I32
    lib.qknorm_strerror.argtypes = [ctypes.c_int]
    lib.qknorm_strerror.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().qknorm_strerror(int(code)).decode()


def abi_version() -> int:
    return int(load().qknorm_abi_version())


# ----------------------------------------------------------------- marshal --

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return QKNORM_F32
    if t.dtype == torch.bfloat16:
        return QKNORM_BF16
    if t.dtype == torch.float16:
        return QKNORM_F16
    if t.dtype == torch.float8_e4m3fn:
        return QKNORM_FP8_E4M3
    raise ValueError("QK-Norm supports float32, bfloat16, float16 and float8_e4m3fn tensors, "
                     f"not {t.dtype}")


def _rows(qkv):
    """(T, ld) of a [T, ...] tensor whose rows are packed."""
    if not qkv.is_cuda:
        raise ValueError("qkv must be a GPU tensor (the library has no CPU path)")
    if qkv.dim() < 2:
        raise ValueError("qkv must have a leading token dimension and at least one more")
    T = qkv.shape[0]
    row = qkv[0] if T > 0 else qkv.new_empty(qkv.shape[1:])
    if T > 0 and not row.is_contiguous():
        raise ValueError("each qkv row must be contiguous")
    ld = qkv.stride(0) if T > 1 else max(qkv.stride(0), row.numel())
    return T, ld, row.numel()


def _ptr(t, dev=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    if dev is not None and t.device != dev:
        raise ValueError("all tensors must be on the same GPU")
    return t.data_ptr()


def _gamma(g, qkv):
    import torch
    if g is None:
        return None
    want = torch.bfloat16 if qkv.dtype == torch.float8_e4m3fn else qkv.dtype
    if g.dtype != want:
        raise ValueError(f"gamma must be {want} for {qkv.dtype} activations")
    if not g.is_contiguous():
        raise ValueError("gamma must be contiguous")
    return _ptr(g, qkv.device)


def _stream(stream, dev):
    if stream is None:
        import torch
        return torch.cuda.current_stream(dev).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _raise(rc: int, what: str):
    if rc == QKNORM_OK:
        return
    if rc == QKNORM_E_HIP:
        raise QKNormError(rc, what)
    raise ValueError(f"{what}: {strerror(rc)} (code {rc})")


# -------------------------------------------------------------- entry points --

def qknorm_per_head(qkv, hq: int, hkv: int, head_dim: int, gamma_q, gamma_k=None,
                    eps: float = 1e-6, stream=None) -> None:
    """Per-head RMSNorm of the hq Q heads and hkv K heads of each row, in place."""
    T, ld, _ = _rows(qkv)
    rc = load().qknorm_per_head(_ptr(qkv), T, ld, hq, hkv, head_dim, _gamma(gamma_q, qkv),
                                _gamma(gamma_k, qkv), eps, _dtype_code(qkv),
                                _stream(stream, qkv.device))
    _raise(rc, "qknorm_per_head")


def qknorm_layerwise(qkv, wq: int, wk: int, gamma_q, gamma_k=None, eps: float = 1e-6,
                     nshards: int = 1, stream=None) -> None:
    """Layerwise RMSNorm over the whole Q and K widths via nshards partials, in place."""
    T, ld, _ = _rows(qkv)
    rc = load().qknorm_layerwise(_ptr(qkv), T, ld, wq, wk, _gamma(gamma_q, qkv),
                                 _gamma(gamma_k, qkv), eps, nshards, _dtype_code(qkv),
                                 _stream(stream, qkv.device))
    _raise(rc, "qknorm_layerwise")


def _partials(p, qkv):
    import torch
    if p is None:
        return None
    if p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("partials must be contiguous float32 [nshards, T]")
    return _ptr(p, qkv.device)


def qknorm_partial_sumsq(qkv, wq: int, wk: int, nshards: int, part_q, part_k,
                         stream=None) -> None:
    """Shard partial sums of squares into part_q / part_k, float32 [nshards, T]."""
    T, ld, _ = _rows(qkv)
    rc = load().qknorm_partial_sumsq(_ptr(qkv), T, ld, wq, wk, nshards, _partials(part_q, qkv),
                                     _partials(part_k, qkv), _dtype_code(qkv),
                                     _stream(stream, qkv.device))
    _raise(rc, "qknorm_partial_sumsq")


def qknorm_apply_scalar(qkv, wq: int, wk: int, part_q, part_k, norm_wq: int, norm_wk: int,
                        gamma_q, gamma_k=None, eps: float = 1e-6, nparts: int | None = None,
                        stream=None) -> None:
    """Combine nparts partials per token and apply, in place."""
    T, ld, _ = _rows(qkv)
    if nparts is None:
        ref = part_q if part_q is not None else part_k
        nparts = ref.shape[0] if ref is not None else 1
    rc = load().qknorm_apply_scalar(_ptr(qkv), T, ld, wq, wk, _partials(part_q, qkv),
                                    _partials(part_k, qkv), nparts, norm_wq, norm_wk,
                                    _gamma(gamma_q, qkv), _gamma(gamma_k, qkv), eps,
                                    _dtype_code(qkv), _stream(stream, qkv.device))
    _raise(rc, "qknorm_apply_scalar")


__all__ = ["qknorm_per_head", "qknorm_layerwise", "qknorm_partial_sumsq", "qknorm_apply_scalar",
           "strerror", "abi_version", "load", "QKNormError", "QKNORM_F32", "QKNORM_BF16", "QKNORM_F16",
           "QKNORM_FP8_E4M3"]
