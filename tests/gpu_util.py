"""Helpers for the GPU parity tests: device buffers with guard bands,
element-wise comparison with the fp64 oracle, and ulp statistics."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from qk_norm_amd import synth

RTOL = {synth.F32: 1e-5, synth.BF16: 8e-3, synth.F16: 1e-3, synth.F8: 0.125}
# fp16 and E4M3 outputs can be subnormal, where the spacing is fixed
# (2^-24 and 2^-9)
ATOL = {synth.F32: 0.0, synth.BF16: 0.0, synth.F16: 2.0 ** -24, synth.F8: 2.0 ** -9}
GUARD_BYTES = 4096
SENTINEL = 0xA5


def torch_dtype(dtype):
    return {synth.F32: torch.float32, synth.BF16: torch.bfloat16, synth.F16: torch.float16,
            synth.F8: torch.float8_e4m3fn}[dtype]


def host_to_device(a: np.ndarray, dtype, dev="cuda"):
    """numpy storage (float32, uint16 bf16/fp16 bits or uint8 E4M3 bytes) -> torch
    tensor of dtype on the GPU."""
    if dtype == synth.F32:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    elif dtype == synth.F8:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch_dtype(dtype))
    return t.to(dev)


def device_to_host(t, dtype) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == synth.F32:
        return t.numpy().copy()
    if dtype == synth.F8:
        return t.view(torch.uint8).numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


class Guarded:
    """A [rows, cols] tensor inside one allocation with sentinel bytes before and after."""

    def __init__(self, host: np.ndarray, dtype, dev="cuda"):
        self.dtype = dtype
        es = synth.esize(dtype)
        rows, cols = host.shape
        g = GUARD_BYTES // es
        n = rows * cols
        raw = torch.full((2 * GUARD_BYTES + n * es,), SENTINEL, dtype=torch.uint8, device=dev)
        self.raw = raw
        self.g = g
        body = raw[GUARD_BYTES:GUARD_BYTES + n * es].view(torch_dtype(dtype))
        self.t = body.view(rows, cols)
        if n:
            self.t.copy_(host_to_device(host, dtype, dev))

    def guards_intact(self) -> bool:
        r = self.raw
        return bool((r[:GUARD_BYTES] == SENTINEL).all() and (r[-GUARD_BYTES:] == SENTINEL).all())

    def host(self) -> np.ndarray:
        return device_to_host(self.t, self.dtype)


def guarded_f32(n: int, dev="cuda"):
    """A float32 [n] tensor between sentinel guards (for partials)."""
    raw = torch.full((2 * GUARD_BYTES + 4 * n,), SENTINEL, dtype=torch.uint8, device=dev)
    body = raw[GUARD_BYTES:GUARD_BYTES + 4 * n].view(torch.float32)
    return raw, body


def raw_guards_intact(raw) -> bool:
    return bool((raw[:GUARD_BYTES] == SENTINEL).all() and (raw[-GUARD_BYTES:] == SENTINEL).all())


def decode(a, dtype):
    return oracle.decode(a, dtype)


def assert_close_to_oracle(got: np.ndarray, y64: np.ndarray, dtype, cols=None, label=""):
    """|g - o| <= rtol |o| (+ atol for fp16 subnormals) element by element (o the
    unrounded fp64 oracle value); where o == 0 the GPU value must be a zero."""
    g = decode(got, dtype)
    if cols is not None:
        g = g[:, cols]
        y64 = y64[:, cols]
    rtol, atol = RTOL[dtype], ATOL[dtype]
    err = np.abs(g - y64)
    bad = (err > rtol * np.abs(y64) + atol) | ((y64 == 0) & (g != 0))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"[{i},{j}] gpu={g[i, j]!r} oracle={y64[i, j]!r}" for i, j in idx)
        raise AssertionError(f"{label}: {int(bad.sum())} elements beyond rtol {rtol}: {detail}")
    nz = y64 != 0
    return float((err[nz] / np.abs(y64[nz])).max()) if nz.any() else 0.0


def gamma_to_device(g, dtype, dev="cuda"):
    """gamma in the storage dtype that goes with activations of `dtype`."""
    return None if g is None else host_to_device(g, synth.gamma_dtype(dtype), dev)


def ordinal(bits: np.ndarray, dtype) -> np.ndarray:
    if dtype == synth.F8:
        b = bits.astype(np.int64)
        return np.where(b & 0x80, -(b & 0x7F), b)
    if dtype in (synth.BF16, synth.F16):
        b = bits.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    b = bits.view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, -(b & 0x7FFFFFFF), b)


def ulp_histogram(got: np.ndarray, ref_rounded: np.ndarray, dtype):
    d = np.abs(ordinal(got, dtype) - ordinal(ref_rounded, dtype))
    vals, counts = np.unique(d, return_counts=True)
    return dict(zip(vals.tolist(), counts.tolist()))


def assert_bytes_equal(a: np.ndarray, b: np.ndarray, label=""):
    if not np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8)):
        raise AssertionError(f"{label}: bytes differ")


def upload_rows(seed, T, ld, dtype, chunk=8192, **kw):
    """A seeded [T, ld] input built chunk by chunk on the GPU (host memory stays
    bounded); any row can be regenerated on its own with synth.make_x(row_start=...)."""
    t = torch.empty((T, ld), dtype=torch_dtype(dtype), device="cuda")
    for r0 in range(0, T, chunk):
        n = min(chunk, T - r0)
        t[r0:r0 + n].copy_(host_to_device(synth.make_x(seed, n, ld, dtype, row_start=r0, **kw), dtype))
    return t


def sample_rows(T, n=40, seed=11):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(rows))


def host_rows(seed, rows, ld, dtype, **kw):
    """The same rows regenerated on the host."""
    return np.concatenate([synth.make_x(seed, 1, ld, dtype, row_start=int(r), **kw) for r in rows])
