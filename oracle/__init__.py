"""fp64 CPU oracle for QK-Norm -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The HIP library never calls it and has no fallback to it.

The arithmetic lives in ``qknorm_oracle.c`` (plain C, fp64, OpenMP over
tokens); this module only marshals numpy arrays.  Every function returns the
fp64 result ``y`` (V and padding columns copied through) and the result rounded
once, to nearest-even, to the I/O dtype ``yr`` (same storage as the input:
float32, uint16 bf16 / fp16 bit patterns, or uint8 FP8 E4M3 bytes).  With
FP8 E4M3 activations gamma is bf16.

Pins (tests/test_oracle_pins.py): unit RMS, scale invariance, the shard-sum
identity, exact brute force on tiny inputs, closed-form rows, per-head vs
layerwise identities, numpy/torch library cross-checks, and rounding against
torch's fp64 -> bf16 conversion.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qknorm_oracle.c")
# QKNORM_ORACLE_LIB names another build of the same source to load instead
# (for instance one built with sanitizers, to run the CPU pins under them)
_LIB = os.environ.get("QKNORM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
F16 = 2
F8 = 3      # OCP FP8 E4M3 activations, bf16 gamma

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_per_head.argtypes = [P, I32, I64, I64, I32, I32, I32, P, P, D, P, P]
        lib.oracle_layerwise.argtypes = [P, I32, I64, I64, I64, I64, P, P, D, I32, P, P]
        lib.oracle_partials.argtypes = [P, I32, I64, I64, I64, I64, I32, P, P]
        lib.oracle_apply.argtypes = [P, I32, I64, I64, I64, I64, P, P, I32, D, D, P, P, D, P, P]
        lib.oracle_round.argtypes = [P, I64, I32, P]
        for f in (lib.oracle_per_head, lib.oracle_layerwise, lib.oracle_partials,
                  lib.oracle_apply, lib.oracle_round, lib.oracle_max_threads,
                  lib.oracle_set_threads):
            f.restype = I32
        lib.oracle_set_threads.argtypes = [I32]
        _lib = lib
    return _lib


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> int:
    """Use n OpenMP threads from now on (results do not depend on it); returns
    the count in effect."""
    return int(_load().oracle_set_threads(int(n)))


def _storage(dtype: int):
    if dtype == F32:
        return np.float32
    if dtype in (BF16, F16):
        return np.uint16
    if dtype == F8:
        return np.uint8
    raise ValueError(f"unknown dtype code {dtype}")


def gamma_dtype(dtype: int) -> int:
    """gamma shares the activations' dtype, except bf16 with FP8 E4M3."""
    return BF16 if dtype == F8 else dtype


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=_storage(dtype))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _opt(a, dtype):
    if a is None:
        return None, None
    return _arr(a, dtype)


def _outs(shape, dtype, want_y=True):
    y = np.empty(shape, dtype=np.float64) if want_y else None
    yr = np.empty(shape, dtype=_storage(dtype))
    yp = y.ctypes.data_as(ctypes.c_void_p) if want_y else None
    return y, yr, yp, yr.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: arguments rejected")


def per_head(x, dtype, hq, hkv, head_dim, gamma_q, gamma_k, eps, want_y=True):
    """Per-head QK-Norm of fused rows x[T, ld] (Q heads, then K heads, then V)."""
    x, xp = _arr(x, dtype)
    T, ld = x.shape
    gq_keep, gq = _arr(gamma_q, gamma_dtype(dtype))
    gk_keep, gk = _opt(gamma_k, gamma_dtype(dtype))
    y, yr, yp, yrp = _outs(x.shape, dtype, want_y)
    _check(_load().oracle_per_head(xp, dtype, T, ld, hq, hkv, head_dim, gq, gk,
                                   float(eps), yp, yrp), "per_head")
    return y, yr


def layerwise(x, dtype, wq, wk, gamma_q, gamma_k, eps, nshards=1, want_y=True):
    """Layerwise QK-Norm of fused rows over the full Q and K widths via shard sums."""
    x, xp = _arr(x, dtype)
    T, ld = x.shape
    gq_keep, gq = _opt(gamma_q, gamma_dtype(dtype))
    gk_keep, gk = _opt(gamma_k, gamma_dtype(dtype))
    y, yr, yp, yrp = _outs(x.shape, dtype, want_y)
    _check(_load().oracle_layerwise(xp, dtype, T, ld, wq, wk, gq, gk, float(eps), nshards,
                                    yp, yrp), "layerwise")
    return y, yr


def partials(x, dtype, wq, wk, nshards):
    """fp64 shard sums of squares, each shaped [nshards, T]."""
    x, xp = _arr(x, dtype)
    T, ld = x.shape
    pq = np.empty((nshards, T), dtype=np.float64)
    pk = np.empty((nshards, T), dtype=np.float64)
    _check(_load().oracle_partials(xp, dtype, T, ld, wq, wk, nshards,
                                   pq.ctypes.data_as(ctypes.c_void_p),
                                   pk.ctypes.data_as(ctypes.c_void_p)), "partials")
    return pq, pk


def apply(x, dtype, wq, wk, part_q, part_k, norm_wq, norm_wk, gamma_q, gamma_k, eps,
          want_y=True):
    """Normalise with given partials [nparts, T] and divisors norm_wq, norm_wk."""
    x, xp = _arr(x, dtype)
    T, ld = x.shape
    pq = np.ascontiguousarray(part_q, dtype=np.float64)
    pk = np.ascontiguousarray(part_k, dtype=np.float64)
    nparts = pq.shape[0]
    gq_keep, gq = _opt(gamma_q, gamma_dtype(dtype))
    gk_keep, gk = _opt(gamma_k, gamma_dtype(dtype))
    y, yr, yp, yrp = _outs(x.shape, dtype, want_y)
    _check(_load().oracle_apply(xp, dtype, T, ld, wq, wk, pq.ctypes.data_as(ctypes.c_void_p),
                                pk.ctypes.data_as(ctypes.c_void_p), nparts, float(norm_wq),
                                float(norm_wk), gq, gk, float(eps), yp, yrp), "apply")
    return y, yr


def round_to(v, dtype):
    """Round fp64 values once, to nearest-even, to dtype storage."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=_storage(dtype))
    _check(_load().oracle_round(v.ctypes.data_as(ctypes.c_void_p), v.size, dtype,
                                out.ctypes.data_as(ctypes.c_void_p)), "round")
    return out


def _e4m3_table() -> np.ndarray:
    """fp64 value of every E4M3 byte, from its fields (bias 7, no infinity)."""
    b = np.arange(256)
    e, m = (b >> 3) & 0xF, b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(b & 0x80, -mag, mag)


_E4M3 = _e4m3_table()


def decode(a, dtype):
    """Exact fp64 values of stored elements (bf16 patterns widened)."""
    a = np.asarray(a)
    if dtype == F32:
        return a.astype(np.float64)
    if dtype == F8:
        return _E4M3[np.asarray(a, dtype=np.uint8)]
    if dtype == F16:
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def qkv_proj_per_head(x, w, dtype, hq, hkv, head_dim, gamma_q, gamma_k, eps, norm=True):
    """The QKV projection followed by per-head QK-Norm, in fp64.

    x is [T, K] and w is [N, K] (the projection's weight, one row per output
    column), N = (hq + 2*hkv) * head_dim, both in the storage of `dtype`.
    acc = x @ w^T is taken with numpy's fp64 matmul of the exactly decoded
    values; each Q head (columns h*D, gamma_q) and each K head (columns
    hq*D + h*D, gamma_k) of every row is then normalised over its D values,
    y = acc * gamma / sqrt(sum(acc^2)/D + eps), and the V columns are acc
    itself.  norm=False gives the plain projection.  Returns (y, y rounded
    once to dtype).

    The normalisation is the per-head RMSNorm of per_head() (sglang PR
    "Add turbomind_rms_norm ...", #13189: an RMSNorm over the head dimension),
    applied to the projection's output before any rounding: the fused form
    of the QKV projection ("Explain combined QKV projection ..." lesson,
    "With GQA": one matmul, split into Q, K and V heads).
    """
    xd = decode(x, dtype)
    wd = decode(w, dtype)
    T, N = xd.shape[0], wd.shape[0]
    D = head_dim
    if N != (hq + 2 * hkv) * D:
        raise ValueError("w must have (hq + 2*hkv) * head_dim rows")
    acc = xd @ wd.T
    y = acc.copy()
    if norm:
        gd = gamma_dtype(dtype)
        for c0, nh, g in ((0, hq, gamma_q), (hq * D, hkv, gamma_k)):
            if nh == 0:
                continue
            seg = acc[:, c0:c0 + nh * D].reshape(T, nh, D)
            ms = np.sum(seg * seg, axis=-1, keepdims=True) / D
            y[:, c0:c0 + nh * D] = (seg * decode(g, gd) / np.sqrt(ms + eps)).reshape(T, nh * D)
    return y, round_to(y, dtype)
