"""QKV projection with per-head QK-Norm in its epilogue: the HIP kernel
against the fp64 oracle, through the C ABI.

Tolerance.  The kernel accumulates the K products of each output in fp32
(MFMA, order fixed by the hardware), the oracle in fp64.  The fp32 sum is
within K * 2^-24 * A of the exact one, A = sum_k |x_k w_k| of that output.
  V (and plain) columns: |g - o| <= 8e-3 |o| + 2 K 2^-24 A
  normalised heads: that error passes through y = acc * gamma / rms(acc):
      |g - o| <= 8e-3 |o| + 2 K 2^-24 (|gamma| A / rms + |o| ||A||_2 / ||acc||_2)
  (8e-3 is one bf16 ulp, as for the norm alone; the factor 2 covers the
  norm's own fp32 arithmetic, which is orders of magnitude smaller.)
For fp16 I/O the per-ulp term is 1e-3 |o| + 2^-24 (one fp16 ulp, subnormal
results included), as for the fp16 norm; the accumulation terms are the same.
"""
import numpy as np
import pytest
import torch

import oracle
import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import GUARD_BYTES, Guarded, assert_bytes_equal, gamma_to_device, host_to_device

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
BF16 = synth.BF16
F16 = synth.F16


def make(seed, T, hidden, hq, hkv, D, token_scale=(0.25, 4.0), dtype=BF16):
    """x ~ N(0,1) times a per-token scale; w ~ N(0, 1/hidden) (unit-variance
    outputs); gamma ~ U(0.5, 1.5)."""
    N = (hq + 2 * hkv) * D
    x = synth.make_x(seed, T, hidden, dtype, token_scale=token_scale)
    w = synth.to_dtype(synth.normal(seed + 7, 0, N * hidden).reshape(N, hidden) / np.sqrt(hidden), dtype)
    return x, w, synth.make_gamma(seed, 3, D, dtype), synth.make_gamma(seed, 4, D, dtype)


def _ulp_term(y, dtype):
    return 8e-3 * np.abs(y) if dtype == BF16 else 1e-3 * np.abs(y) + U


def tolerance(x, w, y64, gq, gk, hq, hkv, D, norm=True, dtype=BF16):
    """Per-element bound (see the module docstring)."""
    xd, wd = np.abs(oracle.decode(x, dtype)), np.abs(oracle.decode(w, dtype))
    A = xd @ wd.T
    K = x.shape[1]
    acc = oracle.decode(x, dtype) @ oracle.decode(w, dtype).T
    tol = _ulp_term(y64, dtype) + 2 * K * U * A
    if norm:
        T = x.shape[0]
        for c0, nh, g in ((0, hq, gq), (hq * D, hkv, gk)):
            if nh == 0:
                continue
            sl = slice(c0, c0 + nh * D)
            a = acc[:, sl].reshape(T, nh, D)
            rms = np.sqrt(np.mean(a * a, axis=-1, keepdims=True))
            An = np.linalg.norm(A[:, sl].reshape(T, nh, D), axis=-1, keepdims=True)
            an = np.linalg.norm(a, axis=-1, keepdims=True)
            gd = np.abs(oracle.decode(g, dtype))
            yo = np.abs(y64[:, sl].reshape(T, nh, D))
            extra = 2 * K * U * (gd * A[:, sl].reshape(T, nh, D) / rms + yo * An / an)
            tol[:, sl] = _ulp_term(yo.reshape(T, nh * D), dtype) + extra.reshape(T, nh * D)
    return tol


def run_proj(x, w, hq, hkv, D, gq, gk, eps, ld=None, plain=False, label="", dtype=BF16, ws=False):
    """One call through the C ABI; ws=True takes qknorm_qkv_proj_per_head_ws with
    a workspace of exactly the size asked for, filled with NaN bytes, and
    checks the bytes after it untouched."""
    T, hidden = x.shape
    N = w.shape[0]
    ld = ld or N
    print(f"[proj] {label} T={T} hidden={hidden} hq={hq} hkv={hkv} D={D} ld={ld} plain={plain} "
          f"ws={ws} {synth.DTYPE_NAMES[dtype]}", flush=True)
    xt, wt = host_to_device(x, dtype), host_to_device(w, dtype)
    nan = 0x7FC0 if dtype == BF16 else 0x7E00
    fill = np.full((T, ld), nan, dtype=np.uint16)               # NaN: must be overwritten or kept
    out = Guarded(fill, dtype)
    g1, g2 = gamma_to_device(gq, dtype), gamma_to_device(gk, dtype) if hkv else None
    if ws:
        need = q.qknorm_qkv_proj_workspace_bytes(T, hq, hkv, D)
        space = torch.full((need + GUARD_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
        q.qknorm_qkv_proj_per_head_ws(xt, wt, out.t, hq, hkv, D, g1, g2, eps, plain=plain,
                                      workspace=space[:need] if need else None)
    else:
        q.qknorm_qkv_proj_per_head(xt, wt, out.t, hq, hkv, D, g1, g2, eps, plain=plain)
    torch.cuda.synchronize()
    got = out.host()
    assert out.guards_intact(), "write outside the output"
    if ws:
        assert bool((space[need:] == 0xFF).all()), "write past the workspace"
    assert_bytes_equal(got[:, N:], fill[:, N:], f"{label}: columns past N")
    return got[:, :N]


def check(x, w, hq, hkv, D, gq, gk, eps, got, plain=False, label="", dtype=BF16):
    y64, yr = oracle.qkv_proj_per_head(x, w, dtype, hq, hkv, D, gq, gk if hkv else None, eps,
                                       norm=not plain)
    g = oracle.decode(got, dtype)
    tol = tolerance(x, w, y64, gq, gk, hq, hkv, D, norm=not plain, dtype=dtype)
    bad = ~(np.abs(g - y64) <= tol)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} elements beyond the bound, e.g. [{i},{j}] "
                             f"gpu={g[i, j]!r} oracle={y64[i, j]!r} tol={tol[i, j]!r}")
    exact = np.mean(got == yr)
    assert exact > 0.97, f"{label}: only {exact:.4f} of outputs equal the oracle's rounding"
    return exact


@pytest.mark.parametrize("T,hidden,hq,hkv,D", [
    (1, 64, 2, 1, 128),          # one token, one K step
    (100, 192, 4, 2, 128),       # ragged rows, three K steps
    (333, 512, 3, 1, 64),        # D = 64: N = 320, a half tile of columns
    (130, 256, 32, 8, 128),      # the Qwen3-8B head layout, two row tiles
    (64, 128, 0, 2, 64),         # K heads only
    (48, 64, 5, 0, 64),          # no K or V
    (150, 256, 4, 2, 256),       # D = 256: a head spans the tile's two column waves
    (70, 192, 0, 3, 256),        # D = 256, K heads only
])
def test_fused_projection_against_oracle(T, hidden, hq, hkv, D):
    x, w, gq, gk = make(70 + T, T, hidden, hq, hkv, D)
    eps = synth.eps_f32(1e-6)
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, label="fused")
    check(x, w, hq, hkv, D, gq, gk, eps, got, label=f"fused T={T} K={hidden}")


# Which tile shapes a launch uses depends on the token count and the grid.
# From 17 tokens: 64-row tiles one head wide (four LDS stages; three for
# head_dim 256); above 256 tokens 128-row tiles (the same), up to 512 tokens
# and on to 1024 while they fit one round of the chip's CUs.  Beyond, 256-row
# tiles: a tail of half-width (256 x 128, three stages) tiles is added where
# it fills the CUs better (for head_dim <= 128).  On MI355X's 256 CUs these
# take, in turn: only half-width tiles, only full tiles, and full tiles for
# the first columns with a half-width tail (N = 6144: from column 4864 at
# T = 6000, from column 4096 at T = 4096).
@pytest.mark.parametrize("T,hidden,hq,hkv,D", [
    (640, 256, 32, 8, 128),      # 128-row tiles past 512 tokens: 5 x 48 fit one round
    (400, 320, 8, 2, 256),       # head_dim 256 on 128-row tiles (three stages), five K steps
    (200, 64, 16, 4, 128),       # 64-row tiles, one K step through the four-stage ring
    (768, 256, 32, 8, 128),      # 3 row tiles x 48 half-width tiles: one round
    (2048, 256, 32, 8, 128),     # 8 x 24 full tiles: one round, no tail
    (6000, 256, 32, 8, 128),     # 24 x 19 full tiles, then a tail of 24 x 10 half-width
    (4096, 192, 64, 16, 64),     # head_dim 64: 16 x 16 full tiles, then 16 x 16 half-width
])
def test_full_and_half_width_tiles(T, hidden, hq, hkv, D):
    x, w, gq, gk = make(95 + T, T, hidden, hq, hkv, D)
    eps = synth.eps_f32(1e-6)
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, label="tile shapes")
    check(x, w, hq, hkv, D, gq, gk, eps, got, label=f"tile shapes T={T} K={hidden} D={D}")


def test_plain_projection_and_padding():
    T, hidden, hq, hkv, D = 77, 320, 4, 2, 128
    x, w, gq, gk = make(80, T, hidden, hq, hkv, D)
    N = w.shape[0]
    got = run_proj(x, w, hq, hkv, D, gq, gk, 0.0, ld=N + 40, plain=True, label="plain")
    check(x, w, hq, hkv, D, gq, gk, 0.0, got, plain=True, label="plain")
    got = run_proj(x, w, hq, hkv, D, gq, gk, synth.eps_f32(1e-6), ld=N + 40, label="fused padded")
    check(x, w, hq, hkv, D, gq, gk, synth.eps_f32(1e-6), got, label="fused padded")


@pytest.mark.parametrize("T,hidden,hq,hkv,D", [
    (100, 192, 4, 2, 128),       # ragged rows, three K steps
    (333, 512, 3, 1, 64),        # D = 64, a half tile of columns
    (300, 1024, 32, 8, 128),     # the Qwen3-8B head layout, two row tiles
    (260, 512, 8, 4, 256),       # D = 256
])
def test_fp16_projection_against_oracle(T, hidden, hq, hkv, D):
    # the same kernel with fp16 operands, gamma and output (v_mfma_f32_16x16x32_f16)
    x, w, gq, gk = make(90 + T, T, hidden, hq, hkv, D, dtype=F16)
    eps = synth.eps_f32(1e-6)
    N = w.shape[0]
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, ld=N + 24, label="fp16 fused", dtype=F16)
    check(x, w, hq, hkv, D, gq, gk, eps, got, label=f"fp16 fused T={T} K={hidden}", dtype=F16)
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, plain=True, label="fp16 plain", dtype=F16)
    check(x, w, hq, hkv, D, gq, gk, eps, got, plain=True, label="fp16 plain", dtype=F16)


def test_fused_equals_unfused_up_to_the_intermediate_rounding():
    # projection, then qknorm_per_head on its bf16 output: the fused kernel
    # skips that rounding, so the two agree to within a bf16 ulp or two
    T, hidden, hq, hkv, D = 256, 512, 8, 2, 128
    x, w, gq, gk = make(81, T, hidden, hq, hkv, D)
    eps = synth.eps_f32(1e-6)
    fused = run_proj(x, w, hq, hkv, D, gq, gk, eps, label="fused")
    plain = run_proj(x, w, hq, hkv, D, gq, gk, eps, plain=True, label="plain")
    t = host_to_device(plain, BF16)
    q.qknorm_per_head(t, hq, hkv, D, gamma_to_device(gq, BF16), gamma_to_device(gk, BF16), eps)
    torch.cuda.synchronize()
    unfused = t.cpu().view(torch.int16).numpy().view(np.uint16)
    a, b = oracle.decode(fused, BF16), oracle.decode(unfused, BF16)
    assert np.all(np.abs(a - b) <= 2 * 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-30)
    assert np.array_equal(fused[:, (hq + hkv) * D:], unfused[:, (hq + hkv) * D:]), "V identical"


# Small token counts, 1 to 256, take 64-row tiles (without a workspace).
# Every head_dim, token counts on and off 16-row MFMA blocks, K steps fewer
# than the tiles' four LDS stages (the ring then refetches the last one) or
# not a multiple of them, and each head layout.
@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("T,hidden,hq,hkv,D", [
    (1, 4096, 32, 8, 128),       # a Qwen3-8B decode step
    (8, 4096, 32, 8, 128),
    (32, 4096, 32, 8, 128),
    (17, 320, 4, 2, 128),        # 5 K steps through 4 stages
    (2, 64, 3, 1, 64),           # one K step
    (31, 192, 5, 0, 64),         # no K or V heads
    (15, 448, 0, 3, 64),         # K heads only
    (16, 256, 2, 1, 256),        # head_dim 256
    (29, 576, 1, 2, 256),
    (48, 128, 6, 2, 128),
    (200, 320, 5, 1, 64),        # 64-row tiles: ragged last tile, two heads of 64 per tile
    (256, 256, 2, 2, 256),
])
def test_decode_size_projection(dtype, T, hidden, hq, hkv, D):
    x, w, gq, gk = make(110 + T + D, T, hidden, hq, hkv, D, dtype=dtype)
    eps = synth.eps_f32(1e-6)
    N = w.shape[0]
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, ld=N + 16, label="decode", dtype=dtype)
    check(x, w, hq, hkv, D, gq, gk, eps, got, label=f"decode T={T} K={hidden} D={D}", dtype=dtype)
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, plain=True, label="decode plain", dtype=dtype)
    check(x, w, hq, hkv, D, gq, gk, eps, got, plain=True, label=f"decode plain T={T} D={D}", dtype=dtype)


# Small token counts through the workspace form: up to 8 tokens 16 columns by 4
# slices of K, 9 to 16 tokens 32 columns by 8 slices, 17 to 32 and 33 to 64
# tokens 32 columns with two and four blocks of 16 tokens; above 64 the call
# is the plain one.  K chunks that leave some slices or waves empty, every
# head_dim and head layout, token counts on and off the 16-token blocks.
@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("T,hidden,hq,hkv,D", [
    (1, 4096, 32, 8, 128),       # a Qwen3-8B decode step
    (8, 4096, 32, 8, 128),
    (12, 4096, 32, 8, 128),
    (16, 4096, 32, 8, 128),
    (3, 320, 4, 2, 128),         # 10 K chunks over 4 slices
    (2, 64, 3, 1, 64),           # 2 K chunks over 4 slices: most waves have none
    (9, 64, 1, 1, 64),           # 2 K chunks over 8 slices
    (5, 192, 5, 0, 64),          # no K or V heads
    (15, 448, 0, 3, 64),         # K heads only
    (16, 256, 2, 1, 256),        # head_dim 256
    (7, 576, 1, 2, 256),
    (17, 320, 4, 2, 128),        # two token blocks, the second with one token
    (32, 4096, 32, 8, 128),
    (33, 4096, 32, 8, 128),      # four token blocks, the last three nearly empty
    (64, 4096, 32, 8, 128),
    (50, 64, 1, 1, 64),          # 2 K chunks over the slices
    (40, 576, 1, 2, 256),
    (65, 320, 4, 2, 128),        # above the split range: the workspace is not used
])
def test_decode_size_projection_workspace(dtype, T, hidden, hq, hkv, D):
    x, w, gq, gk = make(310 + T + D, T, hidden, hq, hkv, D, dtype=dtype)
    eps = synth.eps_f32(1e-6)
    N = w.shape[0]
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, ld=N + 16, label="decode ws", dtype=dtype, ws=True)
    check(x, w, hq, hkv, D, gq, gk, eps, got, label=f"decode ws T={T} K={hidden} D={D}", dtype=dtype)
    got = run_proj(x, w, hq, hkv, D, gq, gk, eps, plain=True, label="decode ws plain", dtype=dtype, ws=True)
    check(x, w, hq, hkv, D, gq, gk, eps, got, plain=True, label=f"decode ws plain T={T} D={D}", dtype=dtype)


def test_workspace_size_and_errors_on_the_gpu():
    # a workspace one 256-byte step short, or misaligned, is refused before any
    # launch; the output keeps its fill
    T, hidden, hq, hkv, D = 4, 256, 4, 1, 128
    x, w, gq, gk = make(91, T, hidden, hq, hkv, D)
    xt, wt = host_to_device(x, BF16), host_to_device(w, BF16)
    g1, g2 = gamma_to_device(gq, BF16), gamma_to_device(gk, BF16)
    need = q.qknorm_qkv_proj_workspace_bytes(T, hq, hkv, D)
    assert need == 4 * T * w.shape[0] * 4
    out = torch.zeros(T, w.shape[0], dtype=torch.bfloat16, device="cuda")
    space = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    for bad, code in ((space[:need - 256], q.QKNORM_E_SHAPE), (space[8:need + 8], q.QKNORM_E_ALIGN),
                      (None, q.QKNORM_E_NULLPTR)):
        with pytest.raises(ValueError, match=f"code {code}"):
            q.qknorm_qkv_proj_per_head_ws(xt, wt, out, hq, hkv, D, g1, g2, 1e-6, workspace=bad)
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()


@pytest.mark.parametrize("T,ws", [(200, False), (8, False), (8, True), (13, True), (45, True)],
                         ids=["tiled", "decode", "decode-ws", "decode-ws-32col", "ws-4-token-blocks"])
def test_deterministic_and_graph_replay(T, ws):
    hidden, hq, hkv, D = 256, 4, 1, 128
    x, w, gq, gk = make(82, T, hidden, hq, hkv, D)
    xt, wt = host_to_device(x, BF16), host_to_device(w, BF16)
    g1, g2 = gamma_to_device(gq, BF16), gamma_to_device(gk, BF16)
    out = torch.empty(T, w.shape[0], dtype=torch.bfloat16, device="cuda")
    space = torch.empty(max(q.qknorm_qkv_proj_workspace_bytes(T, hq, hkv, D), 1), dtype=torch.uint8,
                        device="cuda")

    def call():
        if ws:
            q.qknorm_qkv_proj_per_head_ws(xt, wt, out, hq, hkv, D, g1, g2, 1e-6, workspace=space)
        else:
            q.qknorm_qkv_proj_per_head(xt, wt, out, hq, hkv, D, g1, g2, 1e-6)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    call()                                       # the same bits again
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


@pytest.mark.parametrize("T", [4096, 8192])
def test_full_size_qwen3_8b_prefill_every_row(T):
    # [T, 4096] x [6144, 4096]^T, 32 Q + 8 K + 8 V heads of 128, at the two
    # benchmarked token counts (T = 4096 takes full and half-width tiles,
    # T = 8192 full tiles only): every row against the oracle, in chunks
    hidden, hq, hkv, D = 4096, 32, 8, 128
    x, w, gq, gk = make(83, T, hidden, hq, hkv, D)
    eps = synth.eps_f32(1e-6)
    print(f"[proj] full size T={T} hidden={hidden}, every row", flush=True)
    xt, wt = host_to_device(x, BF16), host_to_device(w, BF16)
    out = torch.empty(T, w.shape[0], dtype=torch.bfloat16, device="cuda")
    q.qknorm_qkv_proj_per_head(xt, wt, out, hq, hkv, D, gamma_to_device(gq, BF16),
                               gamma_to_device(gk, BF16), eps)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    del xt, wt, out
    assert not np.isnan(oracle.decode(got, BF16)).any()
    for r0 in range(0, T, 1024):
        rows = slice(r0, min(T, r0 + 1024))
        check(x[rows], w, hq, hkv, D, gq, gk, eps, got[rows], label=f"full size T={T}, rows {r0}..")


def test_rejected_shapes_launch_nothing():
    x = torch.zeros(4, 96, dtype=torch.bfloat16, device="cuda")       # hidden not a multiple of 64
    w = torch.zeros(512, 96, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(4, 512, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="unsupported"):
        q.qknorm_qkv_proj_per_head(x, w, out, 2, 1, 128, g, g)
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(4 * 96, 128, dtype=torch.bfloat16, device="cuda")   # head_dim 96
    with pytest.raises(ValueError, match="unsupported"):
        q.qknorm_qkv_proj_per_head(x, w, out[:, :384], 2, 1, 96, g[:96], g[:96])
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).abs().sum()) == 0
