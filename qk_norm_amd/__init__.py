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

QKNORM_PROJ_PLAIN = 1

EXPORTED = ("qknorm_per_head", "qknorm_layerwise", "qknorm_partial_sumsq",
            "qknorm_apply_scalar", "qknorm_qkv_proj_per_head", "qknorm_qkv_proj_workspace_bytes",
            "qknorm_qkv_proj_per_head_ws", "qknorm_qkv_proj_per_head_noalloc", "qknorm_strerror",
            "qknorm_abi_version")

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
    lib.qknorm_qkv_proj_per_head.argtypes = [P, I64, P, I64, P, I64, I64, I64, I32, I32, I32, P, P,
                                             F, I32, I32, P]
    lib.qknorm_qkv_proj_workspace_bytes.argtypes = [I64, I32, I32, I32]
    lib.qknorm_qkv_proj_workspace_bytes.restype = I64
    lib.qknorm_qkv_proj_per_head_ws.argtypes = [P, I64, P, I64, P, I64, I64, I64, I32, I32, I32, P, P,
                                                F, I32, I32, P, I64, P]
    lib.qknorm_qkv_proj_per_head_noalloc.argtypes = lib.qknorm_qkv_proj_per_head.argtypes
    for name in ("qknorm_per_head", "qknorm_layerwise", "qknorm_partial_sumsq",
                 "qknorm_apply_scalar", "qknorm_qkv_proj_per_head", "qknorm_qkv_proj_per_head_ws",
                 "qknorm_qkv_proj_per_head_noalloc", "qknorm_abi_version"):
        getattr(lib, name).restype = I32
    lib.qknorm_strerror.argtypes = [ctypes.c_int]
    lib.qknorm_strerror.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


_calls_mod = None       # the CPython call module (or its ctypes stand-in)


class _CtypesCalls:
    """The call module's functions through ctypes, for a tree where the module
    is not built (the same library calls, only slower to make)."""

    def __init__(self, lib):
        self.per_head = lib.qknorm_per_head
        self.layerwise = lib.qknorm_layerwise
        self.partial_sumsq = lib.qknorm_partial_sumsq
        self.apply_scalar = lib.qknorm_apply_scalar
        self.qkv_proj_per_head = lib.qknorm_qkv_proj_per_head
        self.qkv_proj_per_head_ws = lib.qknorm_qkv_proj_per_head_ws
        self.qkv_proj_per_head_noalloc = lib.qknorm_qkv_proj_per_head_noalloc

    @staticmethod
    def per_head_t(*_):
        return None

    @staticmethod
    def layerwise_t(*_):
        return None


def _calls():
    """The functions that call the C ABI: `_qknorm_fast` (qk_norm_amd/csrc/pyfast.cpp),
    which converts the Python ints and floats itself and, for the common case of
    contiguous GPU tensors, reads the tensors itself too; or ctypes."""
    global _calls_mod
    if _calls_mod is None:
        lib = load()
        try:
            from . import _qknorm_fast as mod
        except ImportError:
            mod = _CtypesCalls(lib)
        else:
            import torch
            if _CODES is None:
                _torch_tables()
            mod.setup(_raw_stream, torch.Tensor)
        _calls_mod = mod
    return _calls_mod


def strerror(code: int) -> str:
    return load().qknorm_strerror(int(code)).decode()


def abi_version() -> int:
    return int(load().qknorm_abi_version())


# ----------------------------------------------------------------- marshal --

# Everything below runs on every call, so it sticks to cheap tensor
# attributes (shape, stride, dtype, device index) and the raw stream handle.

_CODES = None           # torch dtype -> (dtype code, gamma dtype)
_raw_stream = None      # device index -> current hipStream_t as an int


def _torch_tables():
    global _CODES, _raw_stream
    import torch
    _CODES = {torch.float32: (QKNORM_F32, torch.float32),
              torch.bfloat16: (QKNORM_BF16, torch.bfloat16),
              torch.float16: (QKNORM_F16, torch.float16),
              torch.float8_e4m3fn: (QKNORM_FP8_E4M3, torch.bfloat16)}
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    _raw_stream = raw if raw is not None else (lambda i: torch.cuda.current_stream(i).cuda_stream)


def _dtype_code(t) -> int:
    if _CODES is None:
        _torch_tables()
    try:
        return _CODES[t.dtype][0]
    except KeyError:
        raise ValueError("QK-Norm supports float32, bfloat16, float16 and float8_e4m3fn tensors, "
                         f"not {t.dtype}") from None


def _rows(qkv):
    """(T, ld, device index) of a [T, ...] GPU tensor whose rows are packed."""
    if not qkv.is_cuda:
        raise ValueError("qkv must be a GPU tensor (the library has no CPU path)")
    if qkv.is_contiguous() and qkv.dim() >= 2:
        T = qkv.shape[0]
        if T > 0:                # rows back to back: the pitch is the row's size
            return T, qkv.numel() // T, qkv.get_device()
    shape, stride = qkv.shape, qkv.stride()
    if len(shape) < 2:
        raise ValueError("qkv must have a leading token dimension and at least one more")
    T = shape[0]
    row = 1                      # elements per row, and the check that they are packed
    for n, st in zip(reversed(shape[1:]), reversed(stride[1:])):
        if T > 0 and n != 1 and st != row:
            raise ValueError("each qkv row must be contiguous")
        row *= n
    ld = stride[0] if T > 1 else max(stride[0], row)
    return T, ld, qkv.get_device()


def _ptr(t, dev):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    if t.get_device() != dev:
        raise ValueError("all tensors must be on the same GPU")
    return t.data_ptr()


def _gamma(g, qkv, dev):
    if g is None:
        return None
    if _CODES is None:
        _torch_tables()
    want = _CODES[qkv.dtype][1] if qkv.dtype in _CODES else qkv.dtype
    if g.dtype != want:
        raise ValueError(f"gamma must be {want} for {qkv.dtype} activations")
    if not g.is_contiguous():
        raise ValueError("gamma must be contiguous")
    return _ptr(g, dev)


def _stream(stream, dev):
    if stream is None:
        if _raw_stream is None:
            _torch_tables()
        return _raw_stream(dev)
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
    c = _calls_mod or _calls()
    rc = c.per_head_t(qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps, stream)
    if rc is None:               # not the common case: the full checks, in Python
        T, ld, dev = _rows(qkv)
        rc = c.per_head(qkv.data_ptr(), T, ld, hq, hkv, head_dim, _gamma(gamma_q, qkv, dev),
                        _gamma(gamma_k, qkv, dev), eps, _dtype_code(qkv), _stream(stream, dev))
    if rc:
        _raise(rc, "qknorm_per_head")


def qknorm_layerwise(qkv, wq: int, wk: int, gamma_q, gamma_k=None, eps: float = 1e-6,
                     nshards: int = 1, stream=None) -> None:
    """Layerwise RMSNorm over the whole Q and K widths via nshards partials, in place."""
    c = _calls_mod or _calls()
    rc = c.layerwise_t(qkv, wq, wk, gamma_q, gamma_k, eps, nshards, stream)
    if rc is None:               # not the common case: the full checks, in Python
        T, ld, dev = _rows(qkv)
        rc = c.layerwise(qkv.data_ptr(), T, ld, wq, wk, _gamma(gamma_q, qkv, dev),
                         _gamma(gamma_k, qkv, dev), eps, nshards, _dtype_code(qkv), _stream(stream, dev))
    if rc:
        _raise(rc, "qknorm_layerwise")


def _partials(p, dev):
    import torch
    if p is None:
        return None
    if p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("partials must be contiguous float32 [nshards, T]")
    return _ptr(p, dev)


def qknorm_partial_sumsq(qkv, wq: int, wk: int, nshards: int, part_q, part_k,
                         stream=None) -> None:
    """Shard partial sums of squares into part_q / part_k, float32 [nshards, T]."""
    T, ld, dev = _rows(qkv)
    rc = _calls().partial_sumsq(qkv.data_ptr(), T, ld, wq, wk, nshards,
                                               _partials(part_q, dev), _partials(part_k, dev),
                                               _dtype_code(qkv), _stream(stream, dev))
    _raise(rc, "qknorm_partial_sumsq")


def qknorm_apply_scalar(qkv, wq: int, wk: int, part_q, part_k, norm_wq: int, norm_wk: int,
                        gamma_q, gamma_k=None, eps: float = 1e-6, nparts: int | None = None,
                        stream=None) -> None:
    """Combine nparts partials per token and apply, in place."""
    T, ld, dev = _rows(qkv)
    if nparts is None:
        ref = part_q if part_q is not None else part_k
        nparts = ref.shape[0] if ref is not None else 1
    rc = _calls().apply_scalar(qkv.data_ptr(), T, ld, wq, wk,
                                              _partials(part_q, dev), _partials(part_k, dev),
                                              nparts, norm_wq, norm_wk, _gamma(gamma_q, qkv, dev),
                                              _gamma(gamma_k, qkv, dev), eps, _dtype_code(qkv),
                                              _stream(stream, dev))
    _raise(rc, "qknorm_apply_scalar")


def _matrix(t, dev, what):
    """(pointer, row pitch) of a 2-d GPU tensor with contiguous rows."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{what} must be a 2-d tensor with contiguous rows")
    return _ptr(t, dev), t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _proj_args(x, w, qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps, plain):
    """The C ABI's arguments of a projection call up to `dtype` (the stream is
    added by the caller)."""
    if not qkv.is_cuda:
        raise ValueError("qkv must be a GPU tensor (the library has no CPU path)")
    dev = qkv.get_device()
    xp, ldx = _matrix(x, dev, "x")
    wp, ldw = _matrix(w, dev, "w")
    op, ld = _matrix(qkv, dev, "qkv")
    if x.dtype != qkv.dtype or w.dtype != qkv.dtype:
        raise ValueError("x, w and qkv must share the dtype")
    if x.shape[0] != qkv.shape[0] or x.shape[1] != w.shape[1]:
        raise ValueError("x [T, hidden], w [N, hidden] and qkv [T, >= N] do not match")
    return dev, (xp, ldx, wp, ldw, op, ld, x.shape[0], x.shape[1], hq, hkv, head_dim,
                 None if plain else _gamma(gamma_q, qkv, dev), None if plain else _gamma(gamma_k, qkv, dev),
                 eps, QKNORM_PROJ_PLAIN if plain else 0, _dtype_code(qkv))


def qknorm_qkv_proj_per_head(x, w, qkv, hq: int, hkv: int, head_dim: int, gamma_q=None,
                             gamma_k=None, eps: float = 1e-6, plain: bool = False,
                             stream=None) -> None:
    """qkv[:, :N] = x @ w.T with each Q and K head RMS-normalised in the epilogue.

    x [T, hidden], w [N, hidden] (N = (hq + 2*hkv) * head_dim) and qkv [T, >= N],
    all bfloat16 or all float16 (gamma too) on one GPU; plain=True gives the
    projection alone.
    """
    dev, args = _proj_args(x, w, qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps, plain)
    rc = _calls().qkv_proj_per_head(*args, _stream(stream, dev))
    _raise(rc, "qknorm_qkv_proj_per_head")


def qknorm_qkv_proj_workspace_bytes(T: int, hq: int, hkv: int, head_dim: int) -> int:
    """Bytes of workspace qknorm_qkv_proj_per_head_ws needs (0: none)."""
    n = int(load().qknorm_qkv_proj_workspace_bytes(int(T), int(hq), int(hkv), int(head_dim)))
    if n < 0:
        _raise(n, "qknorm_qkv_proj_workspace_bytes")
    return n


def qknorm_qkv_proj_per_head_ws(x, w, qkv, hq: int, hkv: int, head_dim: int, gamma_q=None,
                                gamma_k=None, eps: float = 1e-6, plain: bool = False,
                                workspace=None, stream=None) -> None:
    """qknorm_qkv_proj_per_head with a workspace: a GPU tensor of at least
    qknorm_qkv_proj_workspace_bytes(T, hq, hkv, head_dim) bytes, contiguous, on
    qkv's device, that no other call uses meanwhile (None where that is 0)."""
    dev, args = _proj_args(x, w, qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps, plain)
    if workspace is None:
        wsp, nbytes = None, 0
    else:
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        wsp, nbytes = _ptr(workspace, dev), workspace.numel() * workspace.element_size()
    rc = _calls().qkv_proj_per_head_ws(*args, wsp, nbytes, _stream(stream, dev))
    _raise(rc, "qknorm_qkv_proj_per_head_ws")


def qknorm_qkv_proj_per_head_noalloc(x, w, qkv, hq: int, hkv: int, head_dim: int, gamma_q=None,
                                     gamma_k=None, eps: float = 1e-6, plain: bool = False,
                                     stream=None) -> None:
    """qknorm_qkv_proj_per_head_ws with the library's own per-GPU scratch in
    place of a workspace (nothing allocated; calls that overlap on one GPU race)."""
    dev, args = _proj_args(x, w, qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps, plain)
    rc = _calls().qkv_proj_per_head_noalloc(*args, _stream(stream, dev))
    _raise(rc, "qknorm_qkv_proj_per_head_noalloc")


__all__ = ["qknorm_per_head", "qknorm_qkv_proj_per_head", "qknorm_qkv_proj_per_head_ws",
           "qknorm_qkv_proj_workspace_bytes", "qknorm_qkv_proj_per_head_noalloc", "qknorm_layerwise", "qknorm_partial_sumsq", "qknorm_apply_scalar",
           "strerror", "abi_version", "load", "QKNormError", "QKNORM_F32", "QKNORM_BF16", "QKNORM_F16",
           "QKNORM_FP8_E4M3"]
