"""Seeded, counter-based synthetic inputs for the QK-Norm workloads.

This module generates *inputs only*: it holds none of the normalisation
arithmetic and is the one piece of code that both the fp64 oracle tests and
the HIP path's tests and bench use.

Random numbers
--------------
Every uniform draw is SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): the i-th output of a stream
with state ``key`` is ``mix(key + (i + 1) * 0x9E3779B97F4A7C15)`` with the
published mixing function below.  Being a pure function of ``(key, i)``, any
element can be regenerated on its own, so a test can rebuild one row of a
32768-row tensor without making the rest.

Streams (the 8-bit ``stream`` id goes into the key):
  0  activations x          (normal, Box-Muller over counter pairs)
  1  per-token scale s_t     (uniform)
  2  outlier-column keys     (uniform; the smallest k keys are the outliers)
  3  gamma for Q             (uniform)
  4  gamma for K             (uniform)

Value structure (the workloads of the five benchmark cases):
  x[t, c] = round_to_dtype( z[t, c] * (20 if c is an outlier column else 1) * s_t )
with z ~ N(0, 1), s_t ~ U(lo, hi) or 1, and gamma = round_to_dtype(U(0.5, 1.5)).
Rounding to bf16 is round-to-nearest-even taken directly from the fp64 value
(no intermediate fp32 step); fp32 and fp16 use numpy's own RNE casts (numpy
rounds fp64 to fp16 directly).

bf16 and fp16 arrays are returned as ``np.uint16`` bit patterns, FP8 E4M3 as
``np.uint8`` bytes (nearest-even, magnitudes past 448 saturate to 448).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F32 = 0
BF16 = 1
F16 = 2
F8 = 3      # OCP FP8 E4M3 activations; gamma stays bf16
DTYPE_NAMES = {F32: "f32", BF16: "bf16", F16: "f16", F8: "fp8e4m3"}


def gamma_dtype(dtype: int) -> int:
    """Storage dtype of gamma: the activations' own, except bf16 with FP8."""
    return BF16 if dtype == F8 else dtype


def esize(dtype: int) -> int:
    return {F32: 4, BF16: 2, F16: 2, F8: 1}[dtype]

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (in place on a uint64 array)."""
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, stream: int) -> np.uint64:
    """State of the SplitMix64 stream ``stream`` for ``seed``."""
    base = np.array([(int(seed) * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    base ^= np.uint64((int(stream) & 0xFF) << 56)
    return _mix(base)[0]


def _uniform_span(key: np.uint64, start: int, count: int) -> np.ndarray:
    """Uniforms in (0, 1) for counters start .. start+count-1 (53-bit, centred)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = key + i * _GOLDEN
        _mix(z)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def uniform(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    key = stream_key(seed, stream)
    return _uniform_span(key, start, count)


def _normal_span(key: np.uint64, start: int, count: int) -> np.ndarray:
    """N(0,1) for element indices start .. start+count-1.

    Element i uses the counter pair (2*(i//2), 2*(i//2)+1): radius from the
    first, angle from the second; even i takes the cosine, odd i the sine.
    """
    p0 = start // 2
    p1 = (start + count + 1) // 2
    npairs = p1 - p0
    u = _uniform_span(key, 2 * p0, 2 * npairs)
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * math.pi * u2
    out = np.empty(2 * npairs, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    off = start - 2 * p0
    return out[off:off + count]


def normal(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    key = stream_key(seed, stream)
    if count <= _CHUNK:
        return _normal_span(key, start, count)
    out = np.empty(count, dtype=np.float64)
    spans = [(s, min(_CHUNK, count - s)) for s in range(0, count, _CHUNK)]

    def work(sp):
        s, n = sp
        out[s:s + n] = _normal_span(key, start + s, n)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, spans))
    return out


def round_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, round to nearest, ties to even, in one step."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # below bf16's normal range the quantum is fixed
    q = np.rint(np.ldexp(v, 8 - e))          # rint: ties to even
    r = np.ldexp(q, e - 8)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)             # exact: r has <= 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_e4m3_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> OCP E4M3 bytes: nearest, ties to even, in one step; 4 significant
    bits, fixed spacing 2^-9 below 2^-6, saturation at +-448 (no infinity)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 512.0)         # anything above 448 saturates below
    _, e = np.frexp(a)                       # a = m * 2**e, 0.5 <= m < 1
    e = np.maximum(e, -5)
    r = np.minimum(np.ldexp(np.rint(np.ldexp(a, 4 - e)), e - 4), 448.0)
    rm, re = np.frexp(r)
    normal = (re - 1 + 7) * 8 + (np.ldexp(rm, 4) - 8)
    code = np.where(r < 2.0 ** -6, np.ldexp(r, 9), normal).astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def to_dtype(v: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == BF16:
        return round_bf16_bits(v)
    if dtype == F16:
        # numpy rounds fp64 -> binary16 directly, nearest-even
        with np.errstate(over="ignore"):
            return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)
    if dtype == F8:
        return round_e4m3_bits(v)
    raise ValueError(f"unknown dtype code {dtype}")


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_columns(seed: int, ncols: int, frac: float) -> np.ndarray:
    """The round(frac*ncols) columns with the smallest stream-2 keys, sorted."""
    k = int(round(frac * ncols))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    keys = uniform(seed, 2, ncols)
    return np.sort(np.argsort(keys, kind="stable")[:k]).astype(np.int64)


@dataclass
class Problem:
    """One seeded QK-Norm problem on fused rows ``x[T, ld]``.

    Columns [0, wq) are Q, [wq, wq+wk) are K, the rest (V, padding) must stay
    bit-identical.  For per-head work wq = hq*D and wk = hkv*D.
    """
    name: str
    dtype: int
    T: int
    ld: int
    wq: int
    wk: int
    x: np.ndarray                 # [T, ld] float32 or uint16 (bf16 bits)
    gamma_q: np.ndarray
    gamma_k: np.ndarray | None
    eps: float                    # the fp32 value handed to the library
    hq: int = 0
    hkv: int = 0
    head_dim: int = 0
    nshards: int = 1
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def esize(self) -> int:
        return esize(self.dtype)


def make_x(seed: int, T: int, ncols: int, dtype: int, *, token_scale=None,
           outlier_frac: float = 0.0, outlier_mult: float = 20.0,
           row_start: int = 0) -> np.ndarray:
    """x[t, c] for rows row_start .. row_start+T-1 of a seeded [*, ncols] tensor."""
    z = normal(seed, 0, T * ncols, start=row_start * ncols).reshape(T, ncols)
    if outlier_frac > 0.0:
        cols = outlier_columns(seed, ncols, outlier_frac)
        z[:, cols] *= outlier_mult
    if token_scale is not None:
        lo, hi = token_scale
        s = lo + (hi - lo) * uniform(seed, 1, T, start=row_start)
        z *= s[:, None]
    return to_dtype(z, dtype)


def make_gamma(seed: int, stream: int, n: int, dtype: int) -> np.ndarray:
    """gamma = U(0.5, 1.5), stored in the gamma dtype that goes with `dtype`."""
    return to_dtype(0.5 + uniform(seed, stream, n), gamma_dtype(dtype))


def eps_f32(eps: float) -> float:
    """The fp64 value of eps after it has been passed as a C float."""
    return float(np.float32(eps))


# ---------------------------------------------------------------------------
# The five benchmark workloads.
# ---------------------------------------------------------------------------

def per_head_problem(name, seed, dtype, T, hq, hkv, D, ld=None, *, token_scale=None,
                     outlier_frac=0.0, eps=1e-6, row_start=0) -> Problem:
    ld = ld if ld is not None else (hq + 2 * hkv) * D
    x = make_x(seed, T, ld, dtype, token_scale=token_scale, outlier_frac=outlier_frac,
               row_start=row_start)
    gq = make_gamma(seed, 3, D, dtype)
    gk = make_gamma(seed, 4, D, dtype) if hkv > 0 else None
    return Problem(name=name, dtype=dtype, T=T, ld=ld, wq=hq * D, wk=hkv * D, x=x,
                   gamma_q=gq, gamma_k=gk, eps=eps_f32(eps), hq=hq, hkv=hkv,
                   head_dim=D, seed=seed)


def layerwise_problem(name, seed, dtype, T, wq, wk, ld, nshards, *, token_scale=None,
                      outlier_frac=0.0, eps=1e-6, row_start=0) -> Problem:
    x = make_x(seed, T, ld, dtype, token_scale=token_scale, outlier_frac=outlier_frac,
               row_start=row_start)
    gq = make_gamma(seed, 3, wq, dtype)
    gk = make_gamma(seed, 4, wk, dtype) if wk > 0 else None
    return Problem(name=name, dtype=dtype, T=T, ld=ld, wq=wq, wk=wk, x=x,
                   gamma_q=gq, gamma_k=gk, eps=eps_f32(eps), nshards=nshards, seed=seed)


def small_fused_f32(seed: int = 1) -> Problem:
    """Per-head, fp32: [4, (16+2*4)*128], Hq=16, Hkv=4, D=128, N(0,1)."""
    return per_head_problem("fused_rows_per_head_f32_T4", seed, F32, 4, 16, 4, 128)


def standalone_heads(T: int = 4096, H: int = 48, seed: int = 2, dtype: int = BF16) -> Problem:
    """Per-head, bf16, standalone [T, H, 128]; N(0,1) times per-token U(0.1, 10)."""
    return per_head_problem(f"standalone_per_head_{DTYPE_NAMES[dtype]}_T{T}_H{H}", seed, dtype, T, H,
                            0, 128, token_scale=(0.1, 10.0))


def fused_gqa_rows(T: int = 8192, seed: int = 3) -> Problem:
    """Fused GQA per-head, bf16: [T, 6144] = Q 32x128 | K 8x128 | V 8x128."""
    return per_head_problem(f"fused_gqa_per_head_bf16_T{T}", seed, BF16, T, 32, 8, 128)


def layerwise_rows(T: int = 256, seed: int = 4) -> Problem:
    """Layerwise via 8 shard partials, bf16: [T, 6144], Q 4096, K 1024, 1% outliers x20."""
    return layerwise_problem(f"layerwise_rows_bf16_T{T}", seed, BF16, T, 4096, 1024, 6144, 8,
                             outlier_frac=0.01)


def prefill_rows(T: int = 32768, seed: int = 5, mode: str = "layerwise", row_start: int = 0,
                 dtype: int = BF16) -> Problem:
    """Large prefill: [T, 10240], Hq=64, Hkv=8, D=128; outliers x20 and per-token U(0.1, 10).

    Per-head and layerwise share x (same seed); only the gamma widths differ.
    """
    name = DTYPE_NAMES[dtype]
    if mode == "per_head":
        return per_head_problem(f"prefill_per_head_{name}_T{T}", seed, dtype, T, 64, 8, 128,
                                token_scale=(0.1, 10.0), outlier_frac=0.01, row_start=row_start)
    return layerwise_problem(f"prefill_layerwise_{name}_T{T}", seed, dtype, T, 8192, 1024, 10240, 8,
                             token_scale=(0.1, 10.0), outlier_frac=0.01, row_start=row_start)


STANDALONE_SWEEP_T = (1, 16, 128, 1024, 4096)
STANDALONE_SWEEP_H = (16, 32, 48)
FUSED_GQA_SWEEP_T = (1, 8, 64, 512, 8192)
LAYERWISE_SWEEP_T = (1, 4, 32, 256)
