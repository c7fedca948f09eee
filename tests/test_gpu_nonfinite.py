"""Non-finite inputs through the C ABI, against the fp64 oracle.

The pages fix the arithmetic (a sum of squares, a reciprocal square root, two
products) and nothing about NaN or infinity, so both sides take IEEE
arithmetic as it comes: a NaN anywhere in a normalised group makes its sum of
squares NaN and every output of the group NaN; an infinity makes the sum
infinite and the scale zero, so the group's finite values become zeros of
their own sign and the infinity itself NaN (inf * 0).  Groups without a
special value are untouched by it.  Checked for every I/O dtype (E4M3 has NaN
but no infinity), per head and layerwise (fused and two-phase, which must
also agree bit for bit), and for FP8 with gammas large enough that results
saturate at +-448, where the saturating selects must leave NaN as NaN.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import Guarded, assert_bytes_equal, gamma_to_device, ordinal
from test_gpu_layerwise import fused, two_phase

pytestmark = pytest.mark.gpu

DTYPES = [synth.F32, synth.BF16, synth.F16, synth.F8]
IDS = ["f32", "bf16", "f16", "fp8"]

# storage patterns of NaN and of +-infinity per I/O dtype (E4M3: none)
NAN = {synth.F32: np.float32(np.nan), synth.BF16: 0x7FC0, synth.F16: 0x7E00, synth.F8: 0x7F}
POS_INF = {synth.F32: np.float32(np.inf), synth.BF16: 0x7F80, synth.F16: 0x7C00}
NEG_INF = {synth.F32: np.float32(-np.inf), synth.BF16: 0xFF80, synth.F16: 0xFC00}


def check(got, y64, yr, dtype, qk, x, label):
    """NaN exactly where the oracle has NaN; elsewhere the usual bar (fp32:
    1e-5 relative to the fp64 value, zeros where it is zero; 16-bit and FP8:
    at most one ulp from the oracle's own rounding); V bytes untouched."""
    g = oracle.decode(got[:, :qk], dtype)
    o = y64[:, :qk]
    gnan, onan = np.isnan(g), np.isnan(o)
    assert np.array_equal(gnan, onan), \
        f"{label}: NaN at {np.argwhere(gnan != onan)[:5].tolist()} differs from the oracle"
    ok = ~onan
    if dtype == synth.F32:
        err = np.abs(g[ok] - o[ok])
        assert np.all(err <= 1e-5 * np.abs(o[ok])), f"{label}: beyond 1e-5"
        assert np.all(g[ok][o[ok] == 0] == 0), f"{label}: a zero of the oracle is not zero"
    else:
        d = np.abs(ordinal(got[:, :qk], dtype) - ordinal(yr[:, :qk], dtype))
        assert d[ok].max() <= 1, f"{label}: {int((d[ok] > 1).sum())} values beyond one ulp"
    assert_bytes_equal(got[:, qk:], x[:, qk:], f"{label}: V/padding columns")


def _plant(x, dtype, cells):
    x = x.copy()
    for (r, c, kind) in cells:
        x[r, c] = {"nan": NAN, "+inf": POS_INF, "-inf": NEG_INF}[kind][dtype]
    return x


def _scaled_gamma(g, dtype, factor):
    gd = synth.gamma_dtype(dtype)
    return synth.to_dtype(oracle.decode(g, gd) * factor, gd)


def _per_head_cells(dtype, hq, D):
    cells = [(0, 1 * D + 5, "nan"),            # a Q head: all NaN
             (3, 0, "nan")]                     # first element of the row
    if dtype != synth.F8:
        cells += [(1, hq * D + 7, "+inf"),     # a K head: zeros and one NaN
                  (2, 3 * D, "-inf"),           # another Q head, -inf
                  (4, 2 * D + 1, "+inf"), (4, 2 * D + 9, "nan")]   # both in one head
    return cells


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_per_head_nonfinite(dtype):
    hq, hkv, D, T = 4, 2, 128, 6
    ld = (hq + 2 * hkv) * D + 16 // synth.esize(dtype)
    p = synth.per_head_problem(f"nonfinite_per_head_{synth.DTYPE_NAMES[dtype]}", 61, dtype, T, hq, hkv, D, ld)
    p = dataclasses.replace(p, x=_plant(p.x, dtype, _per_head_cells(dtype, hq, D) + [(5, ld - 1, "nan")]))
    print(f"[nonfinite] per-head {p.name}", flush=True)
    buf = Guarded(p.x, dtype)
    q.qknorm_per_head(buf.t, hq, hkv, D, gamma_to_device(p.gamma_q, dtype), gamma_to_device(p.gamma_k, dtype),
                      p.eps)
    torch.cuda.synchronize()
    assert buf.guards_intact()
    y64, yr = oracle.per_head(p.x, dtype, hq, hkv, D, p.gamma_q, p.gamma_k, p.eps)
    assert np.isnan(y64[0, D:2 * D]).all() and not np.isnan(y64[0, :D]).any()   # the reading itself
    check(buf.host(), y64, yr, dtype, (hq + hkv) * D, p.x, p.name)


def test_per_head_nonfinite_fp8_saturating():
    # gammas of 75 to 225: results pass 448 and take the saturating selects, which
    # must not turn a NaN into +-448
    dtype, hq, hkv, D, T = synth.F8, 4, 2, 128, 6
    p = synth.per_head_problem("nonfinite_per_head_fp8_sat", 62, dtype, T, hq, hkv, D)
    p = dataclasses.replace(p, x=_plant(p.x, dtype, _per_head_cells(dtype, hq, D)),
                            gamma_q=_scaled_gamma(p.gamma_q, dtype, 150.0),
                            gamma_k=_scaled_gamma(p.gamma_k, dtype, 150.0))
    print(f"[nonfinite] per-head {p.name}", flush=True)
    buf = Guarded(p.x, dtype)
    q.qknorm_per_head(buf.t, hq, hkv, D, gamma_to_device(p.gamma_q, dtype), gamma_to_device(p.gamma_k, dtype),
                      p.eps)
    torch.cuda.synchronize()
    got = buf.host()
    y64, yr = oracle.per_head(p.x, dtype, hq, hkv, D, p.gamma_q, p.gamma_k, p.eps)
    assert (np.abs(oracle.decode(yr, dtype)[~np.isnan(y64)]) == 448).any(), "no result saturates"
    check(got, y64, yr, dtype, (hq + hkv) * D, p.x, p.name)


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("wq,wk,R", [(1024, 256, 8), (4096, 1024, 8)])
def test_layerwise_nonfinite(dtype, wq, wk, R):
    T = 5
    ld = wq + 2 * wk
    p = synth.layerwise_problem(f"nonfinite_layerwise_{synth.DTYPE_NAMES[dtype]}_{wq}", 63, dtype, T, wq, wk, ld, R)
    cells = [(0, 100, "nan"),                       # Q of row 0 NaN, its K untouched
             (3, wq + wk + 2, "nan")]               # a V column: must come back as it was
    if dtype != synth.F8:
        cells += [(1, wq + 5, "+inf"),              # K of row 1: zeros and one NaN
                  (2, wq - 1, "-inf"), (2, wq + wk - 1, "nan")]
    else:
        cells += [(1, wq + 5, "nan")]
    p = dataclasses.replace(p, x=_plant(p.x, dtype, cells))
    a = fused(p)
    b, _, _ = two_phase(p)
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{p.name}: fused and two-phase differ"
    y64, yr = oracle.layerwise(p.x, dtype, wq, wk, p.gamma_q, p.gamma_k, p.eps, R)
    assert np.isnan(y64[0, :wq]).all() and not np.isnan(y64[0, wq:wq + wk]).any()
    check(a, y64, yr, dtype, wq + wk, p.x, p.name)
