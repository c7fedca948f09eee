"""Tensors past 4 GiB: every kernel addresses rows through 64-bit bases with
32-bit offsets inside a trip or tile, so rows beyond 4 GiB must land where
rows below it do.  The inputs repeat one seeded block of 8192 rows (row r is
block row r % 8192), so sampled rows from both ends are checked against the
oracle, and a row written at a wrapped 32-bit address would show up as an
unnormalised row at the top and a twice-normalised one below it."""
import numpy as np
import pytest
import torch

import oracle
import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import (assert_close_to_oracle, device_to_host, gamma_to_device, host_rows,
                      host_to_device, upload_rows)
from test_gpu_proj import tolerance as proj_tolerance

pytestmark = pytest.mark.gpu

BLOCK = 8192
GIB4 = 1 << 32


def _tiled(seed, T, ld, dtype, **kw):
    block = upload_rows(seed, BLOCK, ld, dtype, **kw)
    # repeat through a same-size integer view (float8 repeats are not
    # implemented everywhere)
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[block.element_size()]
    big = block.view(view).repeat(T // BLOCK, 1).view(block.dtype)
    del block
    return big


def _rows(T):
    # both ends, the 4 GiB boundary's neighbourhood and a spread in between
    rng = np.random.default_rng(17)
    return np.unique(np.concatenate([[0, 1, BLOCK - 1, T // 2, T - 2, T - 1],
                                     rng.choice(T, 24, replace=False)]))


def _gather(t, rows, dtype):
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    return device_to_host(t.view(view)[torch.from_numpy(rows).cuda()].view(t.dtype), dtype)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_per_head_past_4gib():
    dtype, T, H, D = synth.BF16, 64 * BLOCK, 48, 128
    ld, seed = H * D, 71
    print(f"[huge per-head] T={T} H={H} D={D}: {T * ld * 2 / 2**30:.1f} GiB", flush=True)
    x = _tiled(seed, T, ld, dtype, token_scale=(0.1, 10.0))
    assert x.numel() * 2 > GIB4
    g = synth.make_gamma(seed, 3, D, dtype)
    q.qknorm_per_head(x, H, 0, D, gamma_to_device(g, dtype), None, synth.eps_f32(1e-6))
    torch.cuda.synchronize()
    rows = _rows(T)
    xs = host_rows(seed, rows % BLOCK, ld, dtype, token_scale=(0.1, 10.0))
    y64, _ = oracle.per_head(xs, dtype, H, 0, D, g, None, synth.eps_f32(1e-6))
    assert_close_to_oracle(_gather(x, rows, dtype), y64, dtype, label="per-head past 4 GiB")
    # every copy of the block came out the same
    first = x[:BLOCK].clone()
    for b in range(1, T // BLOCK):
        assert torch.equal(x[b * BLOCK:(b + 1) * BLOCK].view(torch.int16), first.view(torch.int16)), \
            f"block {b} differs from block 0"
    del x, first
    _free()


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F8], ids=["bf16", "fp8"])
def test_layerwise_fused_and_two_phase_past_4gib(dtype):
    es = synth.esize(dtype)
    T, wq, wk, ld, R = (64 if es == 1 else 32) * BLOCK, 8192, 1024, 10240, 8
    seed = 72
    print(f"[huge layerwise] {synth.DTYPE_NAMES[dtype]} T={T} ld={ld}: {T * ld * es / 2**30:.1f} GiB twice",
          flush=True)
    a = _tiled(seed, T, ld, dtype, token_scale=(0.1, 10.0))
    assert a.numel() * es > GIB4
    b = a.clone()
    gq = synth.make_gamma(seed, 3, wq, dtype)
    gk = synth.make_gamma(seed, 4, wk, dtype)
    gqd, gkd = gamma_to_device(gq, dtype), gamma_to_device(gk, dtype)
    eps = synth.eps_f32(1e-6)
    q.qknorm_layerwise(a, wq, wk, gqd, gkd, eps, R)
    pq = torch.empty(R, T, dtype=torch.float32, device="cuda")
    pk = torch.empty(R, T, dtype=torch.float32, device="cuda")
    q.qknorm_partial_sumsq(b, wq, wk, R, pq, pk)
    q.qknorm_apply_scalar(b, wq, wk, pq, pk, wq, wk, gqd, gkd, eps)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "fused and two-phase differ"
    del b, pq, pk
    _free()
    rows = _rows(T)
    xs = host_rows(seed, rows % BLOCK, ld, dtype, token_scale=(0.1, 10.0))
    y64, _ = oracle.layerwise(xs, dtype, wq, wk, gq, gk, eps, R)
    got = _gather(a, rows, dtype)
    assert_close_to_oracle(got[:, :wq + wk], y64[:, :wq + wk], dtype, label="layerwise past 4 GiB")
    assert np.array_equal(got[:, wq + wk:], xs[:, wq + wk:]), "V columns changed"
    del a
    _free()


def test_projection_output_past_4gib():
    T, hidden, hq, hkv, D = 44 * BLOCK, 4096, 32, 8, 128
    N = (hq + 2 * hkv) * D
    seed = 73
    print(f"[huge proj] T={T} hidden={hidden} N={N}: output {T * N * 2 / 2**30:.1f} GiB", flush=True)
    x = _tiled(seed, T, hidden, synth.BF16, token_scale=(0.25, 4.0))
    w = synth.to_dtype(synth.normal(seed + 7, 0, N * hidden).reshape(N, hidden) / np.sqrt(hidden),
                       synth.BF16)
    gq, gk = synth.make_gamma(seed, 3, D, synth.BF16), synth.make_gamma(seed, 4, D, synth.BF16)
    eps = synth.eps_f32(1e-6)
    out = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    assert out.numel() * 2 > GIB4
    q.qknorm_qkv_proj_per_head(x, host_to_device(w, synth.BF16), out, hq, hkv, D,
                               gamma_to_device(gq, synth.BF16), gamma_to_device(gk, synth.BF16), eps)
    torch.cuda.synchronize()
    del x
    # Each XCD's tiles start their walk through K at a different step, so two
    # copies of a row can be summed in different orders: the copies are each
    # held to the oracle's bound rather than to each other's bits.  The oracle
    # is computed once per chunk of the repeated block and every row of four
    # blocks is checked against it: the first two, one in the middle and the
    # last, which lies past 4 GiB.
    xs = host_rows(seed, np.arange(BLOCK), hidden, synth.BF16, token_scale=(0.25, 4.0))
    blocks = (0, 1, T // BLOCK // 2, T // BLOCK - 1)
    assert (T // BLOCK - 1) * BLOCK * N * 2 >= GIB4
    got = {b: out[b * BLOCK:(b + 1) * BLOCK].cpu().view(torch.int16).numpy().view(np.uint16)
           for b in blocks}
    del out
    _free()
    for r0 in range(0, BLOCK, 1024):
        rows = slice(r0, r0 + 1024)
        y64, yr = oracle.qkv_proj_per_head(xs[rows], w, synth.BF16, hq, hkv, D, gq, gk, eps)
        tol = proj_tolerance(xs[rows], w, y64, gq, gk, hq, hkv, D)
        for b in blocks:
            g = oracle.decode(got[b][rows], synth.BF16)
            bad = ~(np.abs(g - y64) <= tol)
            assert not bad.any(), \
                f"projection past 4 GiB: block {b} rows {r0}..: {int(bad.sum())} beyond the bound"
            exact = np.mean(got[b][rows] == yr)
            assert exact > 0.97, f"block {b} rows {r0}..: only {exact:.4f} equal the oracle's rounding"
