"""qknorm_qkv_proj_per_head_noalloc, the split decode-size projection on the
library's own per-GPU scratch, through the C ABI: against
qknorm_qkv_proj_per_head_ws (the same kernels on a caller's workspace), bit
for bit, and against the fp64 oracle to the projection tests' bound.  Two
calls in a row, the second with a smaller input (fewer tokens, fewer columns,
another K), so the second call runs on scratch that still holds the first
call's partials."""
import numpy as np
import pytest
import torch

import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import gamma_to_device, host_to_device
from test_gpu_proj import check, make

pytestmark = pytest.mark.gpu
BF16 = synth.BF16

# a Qwen3-8B decode step of 16 tokens (3 MiB of partials), then 3 tokens of a small layer
CASES = [(16, 4096, 32, 8, 128, 401), (3, 320, 4, 2, 128, 402)]


def _call(entry, x, w, hq, hkv, D, gq, gk, eps, plain):
    T, N = x.shape[0], w.shape[0]
    xt, wt = host_to_device(x, BF16), host_to_device(w, BF16)
    out = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    g1, g2 = gamma_to_device(gq, BF16), gamma_to_device(gk, BF16)
    if entry == "noalloc":
        q.qknorm_qkv_proj_per_head_noalloc(xt, wt, out, hq, hkv, D, g1, g2, eps, plain=plain)
    else:
        need = q.qknorm_qkv_proj_workspace_bytes(T, hq, hkv, D)
        space = torch.empty(need, dtype=torch.uint8, device="cuda")
        q.qknorm_qkv_proj_per_head_ws(xt, wt, out, hq, hkv, D, g1, g2, eps, plain=plain, workspace=space)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("plain", [False, True], ids=["fused", "plain"])
def test_noalloc_matches_workspace_form_on_two_calls(plain):
    eps = synth.eps_f32(1e-6)
    for T, hidden, hq, hkv, D, seed in CASES:
        print(f"[noalloc] T={T} hidden={hidden} hq={hq} hkv={hkv} D={D} plain={plain}", flush=True)
        x, w, gq, gk = make(seed, T, hidden, hq, hkv, D)
        got = _call("noalloc", x, w, hq, hkv, D, gq, gk, eps, plain)
        ref = _call("ws", x, w, hq, hkv, D, gq, gk, eps, plain)
        assert np.array_equal(got, ref), f"T={T}: the no-alloc call differs from the workspace call"
        check(x, w, hq, hkv, D, gq, gk, eps, got, plain=plain, label=f"noalloc T={T} plain={plain}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 16 tokens of 130 heads of 128: 32 * 16 * 16640 bytes of partials, past 8 MiB
    T, hidden, hq, hkv, D = 16, 64, 130, 0, 128
    assert q.qknorm_qkv_proj_workspace_bytes(T, hq, hkv, D) > 8 << 20
    x = torch.zeros(T, hidden, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(hq * D, hidden, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(T, hq * D, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(D, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match=f"code {q.QKNORM_E_UNSUPPORTED}"):
        q.qknorm_qkv_proj_per_head_noalloc(x, w, out, hq, hkv, D, g, None, 1e-6)
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()


def test_noalloc_in_a_replayed_graph_with_other_calls_between():
    # captured once, replayed three times; before each replay an eager no-alloc
    # call on other inputs rewrites the scratch, which the replay must not need
    T, hidden, hq, hkv, D = 12, 256, 4, 1, 128
    x, w, gq, gk = make(403, T, hidden, hq, hkv, D)
    x2, w2, gq2, gk2 = make(404, 7, 320, 2, 2, D)
    xt, wt = host_to_device(x, BF16), host_to_device(w, BF16)
    g1, g2 = gamma_to_device(gq, BF16), gamma_to_device(gk, BF16)
    xt2, wt2 = host_to_device(x2, BF16), host_to_device(w2, BF16)
    h1, h2 = gamma_to_device(gq2, BF16), gamma_to_device(gk2, BF16)
    out = torch.empty(T, w.shape[0], dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty(7, w2.shape[0], dtype=torch.bfloat16, device="cuda")
    print("[noalloc] graph replay", flush=True)
    q.qknorm_qkv_proj_per_head_noalloc(xt, wt, out, hq, hkv, D, g1, g2, 1e-6)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            q.qknorm_qkv_proj_per_head_noalloc(xt, wt, out, hq, hkv, D, g1, g2, 1e-6)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        q.qknorm_qkv_proj_per_head_noalloc(xt2, wt2, out2, 2, 2, D, h1, h2, 1e-6)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
