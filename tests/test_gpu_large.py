"""Inputs large enough that the kernels take their multi-trip paths: several
head-groups per wave (per-head), several rows per block (layerwise) and several
row blocks per wave (partial sums).  Checked on sampled rows against the oracle,
with V and padding checked over the whole tensor."""
import numpy as np
import pytest
import torch

import oracle
import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import (assert_bytes_equal, assert_close_to_oracle, device_to_host, gamma_to_device,
                      host_rows, host_to_device, sample_rows, upload_rows)

pytestmark = pytest.mark.gpu


def _gather(t, rows, dtype):
    # index a same-size integer view (row gathers of float8 tensors are not
    # implemented everywhere)
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    return device_to_host(t.view(view)[torch.from_numpy(rows).cuda()].view(t.dtype), dtype)


@pytest.mark.parametrize("layout", ["standalone", "fused"])
def test_per_head_multi_trip(layout):
    # more heads than one pass of the grid covers: the pipelined loop runs
    dtype, D = synth.BF16, 128
    if layout == "standalone":
        T, hq, hkv, ld = 65536, 48, 0, 48 * 128
    else:
        T, hq, hkv, ld = 81920, 32, 8, (32 + 2 * 8) * 128
    print(f"[large per-head] {layout} T={T} ld={ld}", flush=True)
    seed = 61
    x = upload_rows(seed, T, ld, dtype, token_scale=(0.1, 10.0))
    v0 = x[:, (hq + hkv) * D:].clone() if ld > (hq + hkv) * D else None
    gq = synth.make_gamma(seed, 3, D, dtype)
    gk = synth.make_gamma(seed, 4, D, dtype) if hkv else None
    q.qknorm_per_head(x, hq, hkv, D, host_to_device(gq, dtype),
                      host_to_device(gk, dtype) if gk is not None else None, synth.eps_f32(1e-6))
    torch.cuda.synchronize()
    rows = sample_rows(T)
    xs = host_rows(seed, rows, ld, dtype, token_scale=(0.1, 10.0))
    y64, _ = oracle.per_head(xs, dtype, hq, hkv, D, gq, gk, synth.eps_f32(1e-6))
    got = _gather(x, rows, dtype)
    qk = (hq + hkv) * D
    assert_close_to_oracle(got[:, :qk], y64[:, :qk], dtype, label=f"large per-head {layout}")
    if v0 is not None:
        assert torch.equal(x[:, qk:].view(torch.int16), v0.view(torch.int16)), "V changed"


@pytest.mark.parametrize("dtype,T,wq,wk,ld,R", [
    # 262144 rows of [Q 1024 | K 128 | V 128]: the fused kernel's blocks walk
    # ~21 rows each, and phase A has more row blocks than waves in its grid
    (synth.BF16, 262144, 1024, 128, 1280, 8),
    # FP8 rows of [Q 4096 | K 1024 | V 1024]: more rows than the one-wave-per-row
    # kernel has waves on MI355X (32768), so waves take a second row, loaded
    # while the first is stored
    (synth.F8, 40000, 4096, 1024, 6144, 8),
])
def test_layerwise_many_rows_per_block_and_partials_grid_stride(dtype, T, wq, wk, ld, R):
    seed = 62
    print(f"[large layerwise] {synth.DTYPE_NAMES[dtype]} T={T} wq={wq} wk={wk} R={R}", flush=True)
    x0 = upload_rows(seed, T, ld, dtype, outlier_frac=0.01)
    gq = synth.make_gamma(seed, 3, wq, dtype)
    gk = synth.make_gamma(seed, 4, wk, dtype)
    eps = synth.eps_f32(1e-6)
    dq, dk = gamma_to_device(gq, dtype), gamma_to_device(gk, dtype)
    rows = sample_rows(T)
    xs = host_rows(seed, rows, ld, dtype, outlier_frac=0.01)
    # fused
    x = x0.clone()
    q.qknorm_layerwise(x, wq, wk, dq, dk, eps, R)
    torch.cuda.synchronize()
    y64, _ = oracle.layerwise(xs, dtype, wq, wk, gq, gk, eps, R)
    assert_close_to_oracle(_gather(x, rows, dtype)[:, :wq + wk], y64[:, :wq + wk], dtype,
                           label="large layerwise fused")
    assert torch.equal(x[:, wq + wk:].view(torch.uint8), x0[:, wq + wk:].view(torch.uint8))
    # two-phase: same bits everywhere, partials match the oracle on the sampled rows
    x2 = x0.clone()
    pq = torch.empty(R, T, dtype=torch.float32, device="cuda")
    pk = torch.empty(R, T, dtype=torch.float32, device="cuda")
    q.qknorm_partial_sumsq(x2, wq, wk, R, pq, pk)
    q.qknorm_apply_scalar(x2, wq, wk, pq, pk, wq, wk, dq, dk, eps)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.uint8), x.view(torch.uint8)), "two-phase != fused"
    oq, ok = oracle.partials(xs, dtype, wq, wk, R)
    idx = torch.from_numpy(rows).cuda()
    for got, ref in ((pq[:, idx], oq), (pk[:, idx], ok)):
        g = got.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - ref) <= 1e-5 * ref)
