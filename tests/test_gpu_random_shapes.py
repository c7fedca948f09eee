"""Seeded random shapes through the C ABI, against the fp64 oracle.

The other GPU tests pick their shapes by hand (the benchmarked ones, tile and
trip boundaries, the edge cases); these draw them at random from everything
the library accepts, so combinations nobody thought of get run too: any
dtype, head widths of 1 to 64 sixteen-byte vectors, head counts with or
without K, padded rows, ragged token counts, and layerwise shard counts and
widths that land on every kernel (register slots, one wave per row, the
streamed form), and projections of any head layout and token count.  The draw
is fixed (seeded), so a failure names a case that reproduces; each case is
checked to the same bar as the hand-picked ones.
"""
import numpy as np
import pytest

from qk_norm_amd import synth
from test_gpu_layerwise import full_check
from test_gpu_per_head import run_per_head
from test_gpu_proj import check as proj_check, make as proj_make, run_proj

pytestmark = pytest.mark.gpu

DTYPES = (synth.F32, synth.BF16, synth.F16, synth.F8)


def _per_head_cases(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = DTYPES[rng.integers(len(DTYPES))]
        es = synth.esize(dtype)
        vecs = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 48, 64]))   # 16-byte vectors per head
        D = vecs * 16 // es
        hq, hkv = int(rng.integers(0, 13)), int(rng.integers(0, 7))
        if hq + hkv == 0:
            continue
        T = int(rng.choice([1, 2, 3, 7, 31, 64, 100, 257, 300]))
        pad = int(rng.integers(0, 3)) * (16 // es)                          # extra elements per row
        ld = (hq + 2 * hkv) * D + pad
        if T * ld * es > (48 << 20):
            continue
        cases.append((dtype, T, hq, hkv, D, ld, int(rng.integers(1 << 30))))
    return cases


def _layerwise_cases(n, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = DTYPES[rng.integers(len(DTYPES))]
        es = synth.esize(dtype)
        R = int(rng.choice([1, 2, 3, 4, 8, 16]))
        svq = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))           # vectors per Q shard
        svk = int(rng.choice([0, 1, 2, 4, 8, 16, 64]))                      # vectors per K shard
        wq, wk = R * svq * 16 // es, R * svk * 16 // es
        T = int(rng.choice([1, 2, 5, 33, 100, 257]))
        ld = wq + wk + int(rng.integers(0, 3)) * 64 // es                   # V and padding
        if T * ld * es > (48 << 20) or wq * es > (1 << 18):
            continue
        cases.append((dtype, T, wq, wk, R, ld, int(rng.integers(1 << 30))))
    return cases


def _proj_cases(n, seed=2028):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        dtype = (synth.BF16, synth.F16)[rng.integers(2)]
        D = int(rng.choice([64, 128, 256]))
        hq, hkv = int(rng.integers(0, 9)), int(rng.integers(0, 4))
        if hq + hkv == 0:
            hq = 1
        T = int(rng.choice([1, 5, 64, 130, 257, 600]))
        hidden = 64 * int(rng.integers(1, 9))
        pad = 8 * int(rng.integers(0, 3))
        cases.append((dtype, T, hidden, hq, hkv, D, pad, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("dtype,T,hq,hkv,D,ld,seed", _per_head_cases(120))
def test_per_head_random_shape(dtype, T, hq, hkv, D, ld, seed):
    p = synth.per_head_problem(f"random_per_head_{synth.DTYPE_NAMES[dtype]}", seed, dtype, T, hq, hkv, D, ld,
                               token_scale=(0.1, 10.0))
    run_per_head(p)


@pytest.mark.parametrize("dtype,T,wq,wk,R,ld,seed", _layerwise_cases(80))
def test_layerwise_random_shape(dtype, T, wq, wk, R, ld, seed):
    p = synth.layerwise_problem(f"random_layerwise_{synth.DTYPE_NAMES[dtype]}", seed, dtype, T, wq, wk, ld, R,
                                token_scale=(0.1, 10.0), outlier_frac=0.01)
    full_check(p)


@pytest.mark.parametrize("dtype,T,hidden,hq,hkv,D,pad,seed", _proj_cases(24))
def test_projection_random_shape(dtype, T, hidden, hq, hkv, D, pad, seed):
    x, w, gq, gk = proj_make(seed, T, hidden, hq, hkv, D, dtype=dtype)
    eps = synth.eps_f32(1e-6)
    N = w.shape[0]
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, ld=N + pad, label="random", dtype=dtype)
    proj_check(x, w, hq, hkv, D, gq, gk, eps, got, label=f"random projection T={T} K={hidden} D={D}", dtype=dtype)
