"""Per-head QK-Norm: the HIP kernels against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import (Guarded, gamma_to_device, assert_bytes_equal, assert_close_to_oracle, host_to_device,
                      ulp_histogram)

pytestmark = pytest.mark.gpu


def run_per_head(p: synth.Problem, check_ulp=True):
    """Run the GPU per-head path on problem p and check it against the oracle."""
    print(f"[per_head] {p.name} T={p.T} ld={p.ld} hq={p.hq} hkv={p.hkv} D={p.head_dim}", flush=True)
    buf = Guarded(p.x, p.dtype)
    gq = gamma_to_device(p.gamma_q, p.dtype)
    gk = gamma_to_device(p.gamma_k, p.dtype)
    q.qknorm_per_head(buf.t, p.hq, p.hkv, p.head_dim, gq, gk, p.eps)
    torch.cuda.synchronize()
    got = buf.host()
    assert buf.guards_intact(), "write outside the tensor"
    y64, yr = oracle.per_head(p.x, p.dtype, p.hq, p.hkv, p.head_dim, p.gamma_q, p.gamma_k, p.eps)
    qk = p.wq + p.wk
    relmax = assert_close_to_oracle(got[:, :qk], y64[:, :qk], p.dtype, label=p.name)
    assert_bytes_equal(got[:, qk:], p.x[:, qk:], f"{p.name}: V/padding columns")
    if check_ulp and p.dtype in (synth.BF16, synth.F16, synth.F8):
        # fp32 arithmetic is far finer than a 16-bit ulp: at most one ulp from
        # the oracle's own rounding, and nearly always none
        hist = ulp_histogram(got[:, :qk], yr[:, :qk], p.dtype)
        assert max(hist) <= 1, f"{p.name}: ulp histogram {hist}"
        if qk * p.T > 10000:
            assert hist.get(0, 0) / (qk * p.T) > 0.99, f"{p.name}: ulp histogram {hist}"
    return got, relmax


def test_small_fused_rows_f32():
    run_per_head(synth.small_fused_f32())


@pytest.mark.parametrize("H", synth.STANDALONE_SWEEP_H)
@pytest.mark.parametrize("T", synth.STANDALONE_SWEEP_T)
def test_standalone_bf16_sweep(T, H):
    run_per_head(synth.standalone_heads(T=T, H=H))


@pytest.mark.parametrize("T", synth.FUSED_GQA_SWEEP_T)
def test_fused_gqa_bf16_sweep(T):
    run_per_head(synth.fused_gqa_rows(T=T))


ALL_DTYPES = [synth.F32, synth.BF16, synth.F16, synth.F8]


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("D", [8, 16, 32, 64, 128, 256, 512, 1024])
def test_head_dims(dtype, D):
    # every power-of-two head of 16 to 1024 bytes; ragged: 37 rows x (5 Q + 3 K) heads,
    # padding after V
    hb = D * synth.esize(dtype)
    if hb < 16 or hb > 1024:
        pytest.skip(f"{hb}-byte heads are outside the supported 16..1024 bytes")
    p = synth.per_head_problem(f"dims_D{D}", 21, dtype, 37, 5, 3, D, ld=(5 + 6) * D + 64,
                               token_scale=(0.1, 10.0))
    run_per_head(p)


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("T,hq,hkv", [(1, 1, 0), (3, 1, 1), (7, 0, 3), (129, 3, 1), (1000, 7, 2)])
def test_ragged_head_counts(dtype, T, hq, hkv):
    p = synth.per_head_problem(f"ragged_T{T}_{hq}_{hkv}", 22, dtype, T, hq, hkv, 128,
                               ld=(hq + 2 * hkv) * 128 + 16 // synth.esize(dtype))
    run_per_head(p)


# head widths that are not a power of two, and the smallest ones (16 and 32
# bytes): in each dtype, through the lane groups that leave lanes idle
ODD_WIDTHS = [(synth.F32, 4), (synth.F32, 12), (synth.F32, 20), (synth.F32, 100), (synth.F32, 252),
              (synth.BF16, 8), (synth.BF16, 16), (synth.BF16, 24), (synth.BF16, 40),
              (synth.BF16, 48), (synth.BF16, 80), (synth.BF16, 96), (synth.BF16, 112),
              (synth.BF16, 136), (synth.BF16, 192), (synth.BF16, 320), (synth.BF16, 504),
              (synth.F16, 8), (synth.F16, 96), (synth.F16, 200),
              (synth.F8, 16), (synth.F8, 32), (synth.F8, 48), (synth.F8, 80), (synth.F8, 96),
              (synth.F8, 112), (synth.F8, 144), (synth.F8, 1008)]


@pytest.mark.parametrize("dtype,D", ODD_WIDTHS, ids=[f"{synth.DTYPE_NAMES[d]}-D{D}" for d, D in ODD_WIDTHS])
def test_head_widths_any_multiple_of_16_bytes(dtype, D):
    # fused rows with padding (row-wise kernel) and a ragged token count
    pad = 16 // synth.esize(dtype)
    p = synth.per_head_problem(f"odd_D{D}", 25, dtype, 53, 5, 3, D, ld=(5 + 6) * D + pad,
                               token_scale=(0.1, 10.0))
    run_per_head(p)
    # the same heads packed back to back (a standalone [T, H, D] tensor)
    p = synth.per_head_problem(f"odd_packed_D{D}", 26, dtype, 37, 7, 0, D)
    run_per_head(p)


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("hidden", [16, 32, 48, 64, 80, 96, 112, 128])
def test_plain_rmsnorm_small_hidden(dtype, hidden):
    # a plain RMSNorm over [T, hidden] rows with hidden <= 128 (the sizes the
    # PR routes to the head-sized kernel): one head per row
    if (hidden * synth.esize(dtype)) % 16:
        pytest.skip("row not a multiple of 16 bytes")
    p = synth.per_head_problem(f"rms_h{hidden}", 27, dtype, 1001, 1, 0, hidden,
                               token_scale=(0.5, 2.0))
    run_per_head(p)


def test_t0_is_a_noop():
    x = torch.randn(0, 6144, device="cuda").to(torch.bfloat16)
    g = torch.ones(128, device="cuda", dtype=torch.bfloat16)
    q.qknorm_per_head(x, 32, 8, 128, g, g)
    torch.cuda.synchronize()


def test_zero_rows_and_eps_zero_closed_forms():
    # zero head with eps > 0 -> zeros; k equal-magnitude nonzeros with eps = 0 ->
    # gamma * sign * sqrt(D/k) exactly in bf16
    D, H, T = 128, 8, 4
    x = np.zeros((T, H * D))
    roots = {}
    for h, k in enumerate([2, 8, 32, 128, 2, 8, 32, 128]):
        if h == 0:
            continue
        idx = np.arange(0, D, D // k)[:k]
        x[:, h * D + idx] = 0.75 * np.where(np.arange(k) % 2 == 0, 1.0, -1.0)
        roots[h] = (idx, np.sqrt(D / k))
    for dtype in ALL_DTYPES:
        xs = synth.to_dtype(x, dtype)
        g = synth.make_gamma(3, 3, D, dtype)
        for eps in (0.0, synth.eps_f32(1e-6)):
            buf = Guarded(xs, dtype)
            q.qknorm_per_head(buf.t, H, 0, D, gamma_to_device(g, dtype), None, eps)
            torch.cuda.synchronize()
            got = buf.host()
            gd = oracle.decode(got, dtype)
            if eps > 0.0:
                assert np.all(gd[:, :D] == 0.0), "zero head with eps > 0 must stay zero"
            else:
                # 0 / sqrt(0): NaN by IEEE, on both sides
                assert np.all(np.isnan(gd[:, :D]))
                gd[:, :D] = 0.0
            if eps == 0.0:
                want = np.zeros((T, H * D))
                for h, (idx, root) in roots.items():
                    want[:, h * D + idx] = (oracle.decode(g, synth.gamma_dtype(dtype))[idx] *
                                            np.sign(x[:, h * D + idx]) * root)
                # exact in bf16 and fp16 (gamma times a power of two); with E4M3
                # output a bf16 gamma times 2^k can sit on a rounding midpoint,
                # where an fp32 ulp decides, so E4M3 keeps the tolerance checks
                if dtype in (synth.BF16, synth.F16):
                    assert np.array_equal(got[:, D:], synth.to_dtype(want, dtype)[:, D:]), \
                        "closed form, bit exact"
                elif dtype == synth.F8:
                    hist = ulp_histogram(got[:, D:], synth.to_dtype(want, dtype)[:, D:], dtype)
                    assert max(hist) <= 1, f"closed form within one E4M3 ulp: {hist}"
                else:
                    assert np.all(np.abs(gd[:, D:] - want[:, D:]) <= 1e-5 * np.abs(want[:, D:]))
            y64, _ = oracle.per_head(xs, dtype, H, 0, D, g, None, eps)
            assert_close_to_oracle(got[:, D:], y64[:, D:], dtype, label=f"closed forms eps={eps}")


def test_extreme_magnitudes():
    # per-token scales from 1e-8 to 1e8 keep fp32 sums of squares in range
    T, H, D = 16, 4, 128
    z = synth.normal(31, 0, T * H * D).reshape(T, H * D)
    z *= (10.0 ** np.linspace(-8, 8, T))[:, None]
    for dtype in (synth.F32, synth.BF16):
        p = synth.Problem("extreme", dtype, T, H * D, H * D, 0, synth.to_dtype(z, dtype),
                          synth.make_gamma(31, 3, D, dtype), None, synth.eps_f32(1e-6), hq=H,
                          hkv=0, head_dim=D)
        run_per_head(p, check_ulp=False)


def test_extreme_magnitudes_f16():
    # fp16 spans 2^-24 .. 65504: rows of subnormals, rows near the top of the
    # range, and whole heads of the smallest and the largest finite value
    T, H, D = 16, 4, 128
    z = synth.normal(32, 0, T * H * D).reshape(T, H * D)
    z *= (10.0 ** np.linspace(-5, 3.5, T))[:, None]
    z[0, :D] = 2.0 ** -24
    z[1, :D] = -65504.0
    z[1, D:2 * D] = np.where(np.arange(D) % 2 == 0, 65504.0, 2.0 ** -24)
    dtype = synth.F16
    p = synth.Problem("extreme_f16", dtype, T, H * D, H * D, 0, synth.to_dtype(z, dtype),
                      synth.make_gamma(32, 3, D, dtype), None, synth.eps_f32(0.0), hq=H,
                      hkv=0, head_dim=D)
    got, _ = run_per_head(p, check_ulp=False)
    gd = oracle.decode(got, dtype)
    g = oracle.decode(p.gamma_q, dtype)
    assert np.array_equal(gd[0, :D], g), "a head of equal values normalises to gamma"
    assert np.array_equal(gd[1, :D], -g)


@pytest.mark.parametrize("dtype", [synth.F16, synth.F8])
@pytest.mark.parametrize("T", [1, 333, 2048])
def test_fused_gqa_16bit_and_fp8(dtype, T):
    # the fused GQA row of a Qwen3-8B-style layer (32 Q, 8 K, 8 V heads of 128)
    p = synth.per_head_problem(f"gqa_{synth.DTYPE_NAMES[dtype]}_T{T}", 24, dtype, T, 32, 8, 128,
                               token_scale=(0.25, 4.0), outlier_frac=0.01)
    run_per_head(p)


def test_extreme_magnitudes_e4m3():
    # E4M3 spans 2^-9 .. 448: rows of subnormals, rows near the top, a head of
    # the smallest value and a head of the largest
    T, H, D = 16, 4, 128
    dtype = synth.F8
    z = synth.normal(33, 0, T * H * D).reshape(T, H * D)
    z *= (2.0 ** np.linspace(-9, 6, T))[:, None]
    z[0, :D] = 2.0 ** -9
    z[1, :D] = -448.0
    z[1, D:2 * D] = np.where(np.arange(D) % 2 == 0, 448.0, 2.0 ** -9)
    p = synth.Problem("extreme_e4m3", dtype, T, H * D, H * D, 0, synth.to_dtype(z, dtype),
                      synth.make_gamma(33, 3, D, dtype), None, synth.eps_f32(0.0), hq=H,
                      hkv=0, head_dim=D)
    got, _ = run_per_head(p, check_ulp=False)
    _, yr = oracle.per_head(p.x, dtype, H, 0, D, p.gamma_q, None, p.eps)
    # a head of equal values normalises to gamma, rounded to E4M3: within one
    # ulp of the oracle's rounding (a bf16 gamma can sit on an E4M3 midpoint)
    hist = ulp_histogram(got, yr, dtype)
    assert max(hist) <= 1, hist


def test_e4m3_saturates_at_448():
    # gamma = 96 and one nonzero per head: y = 96 * sqrt(128) ~ 1086 > 448, so
    # +-448 (never NaN); the rest of the head is exactly zero
    T, H, D = 8, 6, 128
    dtype = synth.F8
    x = np.zeros((T, H * D))
    x[:, ::D] = np.where(np.arange(T)[:, None] % 2 == 0, 1.5, -0.25) * np.ones((T, H))
    g = synth.to_dtype(np.full(D, 96.0), synth.BF16)
    p = synth.Problem("saturate_e4m3", dtype, T, H * D, H * D, 0, synth.to_dtype(x, dtype), g, None,
                      synth.eps_f32(0.0), hq=H, hkv=0, head_dim=D)
    buf = Guarded(p.x, dtype)
    q.qknorm_per_head(buf.t, H, 0, D, gamma_to_device(g, dtype), None, p.eps)
    torch.cuda.synchronize()
    got = buf.host()
    assert buf.guards_intact()
    _, yr = oracle.per_head(p.x, dtype, H, 0, D, g, None, p.eps)
    assert np.array_equal(got, yr), "saturated E4M3 bytes"
    assert set(np.unique(got[:, ::D]).tolist()) == {0x7E, 0xFE}


@pytest.mark.parametrize("gval", [39.5, 40.0, 41.0, 42.0])
def test_e4m3_range_boundary(gval):
    # one nonzero per head gives |y| = gamma * sqrt(128): 447 (no saturation
    # needed, the range test lets the conversion alone round it), 452.5 and
    # 463.8 (round to 448 either way) and 475 (NaN without saturation).  Q uses
    # this gamma, K a small one, so the two regions take different paths.
    T, hq, hkv, D = 16, 4, 2, 128
    dtype = synth.F8
    x = np.zeros((T, (hq + 2 * hkv) * D))
    x[:, : (hq + hkv) * D: D] = np.where(np.arange(T)[:, None] % 3 == 0, -2.0, 0.375)
    gq = synth.to_dtype(np.full(D, gval), synth.BF16)
    gk = synth.make_gamma(34, 4, D, dtype)
    p = synth.Problem(f"e4m3_boundary_{gval}", dtype, T, x.shape[1], hq * D, hkv * D,
                      synth.to_dtype(x, dtype), gq, gk, synth.eps_f32(0.0), hq=hq, hkv=hkv, head_dim=D)
    buf = Guarded(p.x, dtype)
    q.qknorm_per_head(buf.t, hq, hkv, D, gamma_to_device(gq, dtype), gamma_to_device(gk, dtype), p.eps)
    torch.cuda.synchronize()
    got = buf.host()
    assert buf.guards_intact()
    _, yr = oracle.per_head(p.x, dtype, hq, hkv, D, gq, gk, p.eps)
    assert np.array_equal(got, yr), f"E4M3 bytes at gamma {gval}"
    assert set(np.unique(got[:, : hq * D: D]).tolist()) <= {0x7E, 0xFE}


def test_bitwise_deterministic():
    p = synth.fused_gqa_rows(T=512)
    a, _ = run_per_head(p)
    b, _ = run_per_head(p)
    assert np.array_equal(a, b)


def test_standalone_3d_tensor_and_side_stream():
    p = synth.standalone_heads(T=256, H=32)
    x = host_to_device(p.x, p.dtype).view(256, 32, 128)
    g = gamma_to_device(p.gamma_q, p.dtype)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q.qknorm_per_head(x, 32, 0, 128, g, None, p.eps)
    s.synchronize()
    y64, _ = oracle.per_head(p.x, p.dtype, 32, 0, 128, p.gamma_q, None, p.eps)
    got = x.view(256, 32 * 128).cpu().view(torch.int16).numpy().view(np.uint16)
    assert_close_to_oracle(got, y64, p.dtype, label="3d on a side stream")


def test_rows_with_pitch_view():
    # a [T, (hq+hkv)*D] view into a wider buffer: pitch from stride(0)
    p = synth.fused_gqa_rows(T=64)
    full = host_to_device(p.x, p.dtype)
    view = full[:, : p.wq + p.wk]
    q.qknorm_per_head(view, p.hq, p.hkv, p.head_dim, gamma_to_device(p.gamma_q, p.dtype),
                      gamma_to_device(p.gamma_k, p.dtype), p.eps)
    torch.cuda.synchronize()
    got = full.cpu().view(torch.int16).numpy().view(np.uint16)
    y64, _ = oracle.per_head(p.x, p.dtype, p.hq, p.hkv, p.head_dim, p.gamma_q, p.gamma_k, p.eps)
    assert_close_to_oracle(got[:, : p.wq + p.wk], y64[:, : p.wq + p.wk], p.dtype, label="view")
    assert_bytes_equal(got[:, p.wq + p.wk:], p.x[:, p.wq + p.wk:], "V")


def test_graph_replay_matches_eager():
    p = synth.fused_gqa_rows(T=64)
    src = host_to_device(p.x, p.dtype)
    work = src.clone()
    gq, gk = gamma_to_device(p.gamma_q, p.dtype), gamma_to_device(p.gamma_k, p.dtype)
    q.qknorm_per_head(work, p.hq, p.hkv, p.head_dim, gq, gk, p.eps)
    torch.cuda.synchronize()
    eager = work.clone()
    work.copy_(src)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q.qknorm_per_head(work, p.hq, p.hkv, p.head_dim, gq, gk, p.eps)
    torch.cuda.synchronize()
    for _ in range(4):
        work.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(work.view(torch.int16), eager.view(torch.int16))


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("hq,hkv", [(0, 5), (5, 0), (3, 2)])
def test_rows_without_v_or_padding(dtype, hq, hkv):
    # ld == (hq + hkv) * D: rows back to back; single-region tensors take the
    # flat path, and a K-only tensor must still use gamma_k
    D = 128
    p = synth.per_head_problem(f"packed_{hq}_{hkv}", 23, dtype, 33, hq, hkv, D, ld=(hq + hkv) * D)
    if p.gamma_k is None:
        p.gamma_k = synth.make_gamma(23, 4, D, dtype)
    run_per_head(p)


def test_tensor_calls_take_the_c_marshalling_path():
    # The binding hands contiguous row-major tensors to the call module's
    # per_head_t / layerwise_t, which read the tensors from C.  For those it
    # must launch (return 0, not None) and give the same bytes as the
    # pointer-level call; other layouts must return None (Python path).
    c = q._calls()
    assert type(c).__name__ == "module", "the compiled call module was not loaded"
    p = synth.fused_gqa_rows(T=96)
    src = host_to_device(p.x, p.dtype)
    gq, gk = gamma_to_device(p.gamma_q, p.dtype), gamma_to_device(p.gamma_k, p.dtype)
    a, b = src.clone(), src.clone()
    side = torch.cuda.Stream()
    for stream in (None, side, side.cuda_stream):
        a.copy_(src)
        torch.cuda.synchronize()
        assert c.per_head_t(a, p.hq, p.hkv, p.head_dim, gq, gk, p.eps, stream) == 0
        torch.cuda.synchronize()
        b.copy_(src)
        assert c.per_head(b.data_ptr(), p.T, p.ld, p.hq, p.hkv, p.head_dim, gq.data_ptr(), gk.data_ptr(),
                          p.eps, q._dtype_code(b), torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"stream {stream!r}"
    # layouts the C side leaves to Python
    assert c.per_head_t(a[:, : p.wq + p.wk], p.hq, p.hkv, p.head_dim, gq, gk, p.eps, None) is None
    assert c.per_head_t(a, p.hq, p.hkv, p.head_dim, gq.float(), gk, p.eps, None) is None
    assert c.per_head_t(a.cpu(), p.hq, p.hkv, p.head_dim, gq, gk, p.eps, None) is None
    assert c.per_head_t(a[0], p.hq, p.hkv, p.head_dim, gq, gk, p.eps, None) is None
    # rejected arguments come back as the library's error code, nothing launched
    a.copy_(src)
    torch.cuda.synchronize()
    assert c.per_head_t(a, -1, p.hkv, p.head_dim, gq, gk, p.eps, None) != 0
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), src.view(torch.int16))
    # layerwise on the same rows: tensor call and pointer call agree bit for bit
    lw = synth.layerwise_rows(T=96)
    ls = host_to_device(lw.x, lw.dtype)
    lgq, lgk = gamma_to_device(lw.gamma_q, lw.dtype), gamma_to_device(lw.gamma_k, lw.dtype)
    la, lb = ls.clone(), ls.clone()
    assert c.layerwise_t(la, lw.wq, lw.wk, lgq, lgk, lw.eps, lw.nshards, None) == 0
    assert c.layerwise(lb.data_ptr(), lw.T, lw.ld, lw.wq, lw.wk, lgq.data_ptr(), lgk.data_ptr(), lw.eps, lw.nshards,
                       q._dtype_code(lb), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(la.view(torch.int16), lb.view(torch.int16))
