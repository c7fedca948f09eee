"""Layerwise QK-Norm through shard partials: fused, two-phase and apply-only
paths against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import (Guarded, gamma_to_device, assert_bytes_equal, assert_close_to_oracle, guarded_f32,
                      device_to_host, host_to_device, raw_guards_intact, ulp_histogram)

pytestmark = pytest.mark.gpu

PART_RTOL = 1e-5


def _gammas(p):
    gq = gamma_to_device(p.gamma_q, p.dtype)
    gk = gamma_to_device(p.gamma_k, p.dtype)
    return gq, gk


def fused(p):
    print(f"[layerwise fused] {p.name} T={p.T} wq={p.wq} wk={p.wk} R={p.nshards}", flush=True)
    buf = Guarded(p.x, p.dtype)
    gq, gk = _gammas(p)
    q.qknorm_layerwise(buf.t, p.wq, p.wk, gq, gk, p.eps, p.nshards)
    torch.cuda.synchronize()
    assert buf.guards_intact(), "fused: write outside the tensor"
    return buf.host()


def two_phase(p):
    """partial_sumsq then apply_scalar; returns (output, part_q, part_k) on the host."""
    print(f"[layerwise two-phase] {p.name} T={p.T} wq={p.wq} wk={p.wk} R={p.nshards}", flush=True)
    buf = Guarded(p.x, p.dtype)
    gq, gk = _gammas(p)
    R, T = p.nshards, p.T
    rq, pq = guarded_f32(R * T)
    rk, pk = guarded_f32(R * T)
    pq, pk = pq.view(R, T), pk.view(R, T)
    q.qknorm_partial_sumsq(buf.t, p.wq, p.wk, R, pq if p.wq else None, pk if p.wk else None)
    torch.cuda.synchronize()
    assert buf.guards_intact() and torch.equal(buf.t.cpu().view(torch.uint8).flatten(),
                                               host_to_device(p.x, p.dtype).cpu().view(torch.uint8).flatten()), \
        "partial_sumsq must not modify qkv"
    parts = (pq.cpu().numpy().copy(), pk.cpu().numpy().copy())
    q.qknorm_apply_scalar(buf.t, p.wq, p.wk, pq if p.wq else None, pk if p.wk else None,
                          p.wq, p.wk, gq, gk, p.eps)
    torch.cuda.synchronize()
    assert buf.guards_intact() and raw_guards_intact(rq) and raw_guards_intact(rk)
    return buf.host(), parts[0], parts[1]


def check_against_oracle(p, got, label):
    y64, yr = oracle.layerwise(p.x, p.dtype, p.wq, p.wk, p.gamma_q, p.gamma_k, p.eps, p.nshards)
    qk = p.wq + p.wk
    assert_close_to_oracle(got[:, :qk], y64[:, :qk], p.dtype, label=label)
    assert_bytes_equal(got[:, qk:], p.x[:, qk:], f"{label}: V/padding columns")
    if p.dtype in (synth.BF16, synth.F16, synth.F8):
        # never more than one ulp from the oracle's own rounding (fp32 I/O is
        # held to its 1e-5 relative bound)
        hist = ulp_histogram(got[:, :qk], yr[:, :qk], p.dtype)
        assert max(hist) <= 1, f"{label}: ulp histogram {hist}"


def check_partials(p, pq, pk):
    oq, ok = oracle.partials(p.x, p.dtype, p.wq, p.wk, p.nshards)
    for got, ref, name in ((pq, oq, "Q"), (pk, ok, "K")):
        if ref.size == 0 or (name == "Q" and not p.wq) or (name == "K" and not p.wk):
            continue
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= PART_RTOL * ref), f"{p.name}: {name} partials, max rel {np.max(err / ref)}"


def full_check(p):
    a = fused(p)
    check_against_oracle(p, a, p.name + " fused")
    b, pq, pk = two_phase(p)
    check_partials(p, pq, pk)
    assert np.array_equal(a, b), f"{p.name}: fused and two-phase differ"
    return a


@pytest.mark.parametrize("T", synth.LAYERWISE_SWEEP_T)
def test_layerwise_rows_sweep(T):
    full_check(synth.layerwise_rows(T=T))


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16, synth.F16, synth.F8])
@pytest.mark.parametrize("wq,wk,R,T", [
    (4096, 1024, 1, 33),       # one shard: register path, 8 slots per lane
    (4096, 1024, 2, 17),
    (4096, 1024, 4, 9),
    (4096, 1024, 16, 5),       # more shards than waves
    (8192, 1024, 8, 40),       # large-prefill row width
    (8192, 8192, 1024, 3),     # shard of 8 bf16 = one 16-byte vector
    (16384, 2048, 1, 6),       # too wide for registers: streamed kernel
    (512, 0, 4, 11),           # Q only
    (0, 256, 2, 11),           # K only
    (1536, 384, 3, 21),        # shard count not a power of two
])
def test_layerwise_shapes(dtype, wq, wk, R, T):
    es = synth.esize(dtype)
    if ((wq // R) * es) % 16 or ((wk // R) * es) % 16:
        pytest.skip("shard not a multiple of 16 bytes in this dtype")
    ld = wq + 2 * wk + 64
    p = synth.layerwise_problem(f"lw_{wq}_{wk}_R{R}", 41 + R, dtype, T, wq, wk, ld, R,
                                token_scale=(0.1, 10.0), outlier_frac=0.01)
    full_check(p)


def test_apply_scalar_alone_with_oracle_partials():
    # the apply phase on its own, fed fp32-rounded oracle partials
    p = synth.layerwise_rows(T=32)
    oq, ok = oracle.partials(p.x, p.dtype, p.wq, p.wk, p.nshards)
    fq, fk = oq.astype(np.float32), ok.astype(np.float32)
    buf = Guarded(p.x, p.dtype)
    gq, gk = _gammas(p)
    q.qknorm_apply_scalar(buf.t, p.wq, p.wk, torch.from_numpy(fq).cuda(), torch.from_numpy(fk).cuda(),
                          p.wq, p.wk, gq, gk, p.eps)
    torch.cuda.synchronize()
    got = buf.host()
    y64, _ = oracle.apply(p.x, p.dtype, p.wq, p.wk, fq.astype(np.float64), fk.astype(np.float64),
                          p.wq, p.wk, p.gamma_q, p.gamma_k, p.eps)
    qk = p.wq + p.wk
    assert_close_to_oracle(got[:, :qk], y64[:, :qk], p.dtype, label="apply alone")
    assert_bytes_equal(got[:, qk:], p.x[:, qk:], "V")


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F8], ids=["bf16", "fp8"])
def test_apply_scalar_rank_slice_with_gathered_oracle_partials(dtype):
    """The tensor-parallel form of phase C on its own: this rank holds the
    4096-wide Q slice and the 1024-wide K slice (rank 1 of 3) of vectors that
    are 12288 and 3072 wide.  It receives the three ranks' fp32 partials
    (nparts = 3, not the 8 shards of the fused call) and the full widths as
    divisors.  Partials are the oracle's, rounded to fp32; the output is
    checked against the oracle's apply.  In FP8 this shape takes the
    one-wave-per-row kernel in its apply form."""
    N, rank, T, wq, wk = 3, 1, 37, 4096, 1024
    full = synth.layerwise_problem(f"tp_apply_{synth.DTYPE_NAMES[dtype]}", 57, dtype, T, N * wq, N * wk,
                                   N * (wq + wk), 1, token_scale=(0.1, 10.0), outlier_frac=0.01)
    # rank r's row: [its Q slice | its K slice]
    qs = [full.x[:, r * wq:(r + 1) * wq] for r in range(N)]
    ks = [full.x[:, N * wq + r * wk:N * wq + (r + 1) * wk] for r in range(N)]
    parts_q = np.stack([oracle.partials(np.ascontiguousarray(np.concatenate([qs[r], ks[r]], 1)), dtype,
                                        wq, wk, 1)[0][0] for r in range(N)]).astype(np.float32)
    parts_k = np.stack([oracle.partials(np.ascontiguousarray(np.concatenate([qs[r], ks[r]], 1)), dtype,
                                        wq, wk, 1)[1][0] for r in range(N)]).astype(np.float32)
    x = np.ascontiguousarray(np.concatenate([qs[rank], ks[rank]], 1))
    gq = full.gamma_q[rank * wq:(rank + 1) * wq]
    gk = full.gamma_k[rank * wk:(rank + 1) * wk]
    buf = Guarded(x, dtype)
    q.qknorm_apply_scalar(buf.t, wq, wk, torch.from_numpy(parts_q).cuda(), torch.from_numpy(parts_k).cuda(),
                          N * wq, N * wk, gamma_to_device(gq, dtype), gamma_to_device(gk, dtype), full.eps)
    torch.cuda.synchronize()
    assert buf.guards_intact()
    got = buf.host()
    y64, yr = oracle.apply(x, dtype, wq, wk, parts_q.astype(np.float64), parts_k.astype(np.float64),
                           N * wq, N * wk, gq, gk, full.eps)
    assert_close_to_oracle(got, y64, dtype, label="rank-slice apply")
    hist = ulp_histogram(got, yr, dtype)
    assert max(hist) <= 1, f"rank-slice apply: ulp histogram {hist}"
    # and the slice of the whole-vector layerwise oracle agrees within the same bound
    y_full, _ = oracle.layerwise(full.x, dtype, N * wq, N * wk, full.gamma_q, full.gamma_k, full.eps, 1)
    ref = np.concatenate([y_full[:, rank * wq:(rank + 1) * wq],
                          y_full[:, N * wq + rank * wk:N * wq + (rank + 1) * wk]], 1)
    assert_close_to_oracle(got, ref, dtype, label="rank-slice apply vs whole-vector layerwise")


def test_tensor_parallel_emulation_matches_fused():
    """Each of N = 8 'ranks' owns a contiguous 1/8 slice of Q and of K: it computes
    its one-shard partial, the partials are gathered [N, T], and each rank applies
    with nparts = N and the full widths as divisors.  On one GPU this must equal
    the fused 8-shard kernel bit for bit."""
    p = synth.layerwise_rows(T=64)
    N, T = 8, p.T
    sq, sk = p.wq // N, p.wk // N
    x = host_to_device(p.x, p.dtype)
    gq, gk = _gammas(p)
    part_q = torch.empty(N, T, dtype=torch.float32, device="cuda")
    part_k = torch.empty(N, T, dtype=torch.float32, device="cuda")
    for r in range(N):
        qs = x[:, r * sq:(r + 1) * sq]
        ks = x[:, p.wq + r * sk:p.wq + (r + 1) * sk]
        q.qknorm_partial_sumsq(qs, sq, 0, 1, part_q[r:r + 1], None)
        q.qknorm_partial_sumsq(ks, sk, 0, 1, part_k[r:r + 1], None)
    for r in range(N):
        qs = x[:, r * sq:(r + 1) * sq]
        ks = x[:, p.wq + r * sk:p.wq + (r + 1) * sk]
        q.qknorm_apply_scalar(qs, sq, 0, part_q, None, p.wq, 0, gq[r * sq:(r + 1) * sq], None, p.eps)
        q.qknorm_apply_scalar(ks, sk, 0, part_k, None, p.wk, 0, gk[r * sk:(r + 1) * sk], None, p.eps)
    torch.cuda.synchronize()
    got = x.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = fused(p)
    assert np.array_equal(got, ref), "rank-sliced two-phase differs from the fused kernel"


@pytest.mark.parametrize("dtype", [synth.F16, synth.F8])
def test_tensor_parallel_emulation_other_dtypes(dtype):
    # the same rank-sliced two-phase form in fp16 and E4M3, against the fused
    # kernel (bitwise) and the oracle
    N, T, wq, wk = 8, 48, 4096, 1024
    p = synth.layerwise_problem(f"tp_{synth.DTYPE_NAMES[dtype]}", 52, dtype, T, wq, wk,
                                wq + 2 * wk, N, token_scale=(0.5, 2.0), outlier_frac=0.01)
    sq, sk = wq // N, wk // N
    x = host_to_device(p.x, p.dtype)
    gq, gk = _gammas(p)
    part_q = torch.empty(N, T, dtype=torch.float32, device="cuda")
    part_k = torch.empty(N, T, dtype=torch.float32, device="cuda")
    for r in range(N):
        q.qknorm_partial_sumsq(x[:, r * sq:(r + 1) * sq], sq, 0, 1, part_q[r:r + 1], None)
        q.qknorm_partial_sumsq(x[:, wq + r * sk:wq + (r + 1) * sk], sk, 0, 1, part_k[r:r + 1], None)
    for r in range(N):
        q.qknorm_apply_scalar(x[:, r * sq:(r + 1) * sq], sq, 0, part_q, None, wq, 0,
                              gq[r * sq:(r + 1) * sq], None, p.eps)
        q.qknorm_apply_scalar(x[:, wq + r * sk:wq + (r + 1) * sk], sk, 0, part_k, None, wk, 0,
                              gk[r * sk:(r + 1) * sk], None, p.eps)
    torch.cuda.synchronize()
    got = device_to_host(x, dtype)
    ref = full_check(p)
    assert np.array_equal(got, ref), "rank-sliced two-phase differs from the fused kernel"


def test_e4m3_saturation_fused_and_two_phase():
    # K's gamma of 96 lets |y| reach 96 * sqrt(1024) = 3072 (saturated to 448);
    # Q's small gamma never leaves the range.  Fused and two-phase must both
    # give the oracle's bytes exactly (no NaN).
    T, wq, wk = 40, 4096, 1024
    dtype = synth.F8
    x = synth.normal(61, 0, T * (wq + 2 * wk)).reshape(T, wq + 2 * wk)
    x[:, wq:wq + wk] = 0.0
    x[:, wq + 5] = np.where(np.arange(T) % 2 == 0, 3.0, -0.5)      # one nonzero in K
    x[:, wq + 700] = 0.25
    gq = synth.make_gamma(61, 3, wq, dtype)
    gk = synth.to_dtype(np.full(wk, 96.0), synth.BF16)
    p = synth.Problem("e4m3_saturate_lw", dtype, T, wq + 2 * wk, wq, wk, synth.to_dtype(x, dtype),
                      gq, gk, synth.eps_f32(1e-6), nshards=8)
    a = fused(p)
    b, _, _ = two_phase(p)
    _, yr = oracle.layerwise(p.x, dtype, wq, wk, gq, gk, p.eps, 8)
    assert np.array_equal(a[:, wq:], yr[:, wq:]), "fused: K bytes"
    assert np.array_equal(b[:, wq:], yr[:, wq:]), "two-phase: K bytes"
    assert set(np.unique(a[:, wq + 5]).tolist()) == {0x7E, 0xFE}
    y64, _ = oracle.layerwise(p.x, dtype, wq, wk, gq, gk, p.eps, 8)
    assert_close_to_oracle(a[:, :wq], y64[:, :wq], dtype, label="Q region")
    assert np.array_equal(a, b)


def test_bitwise_deterministic():
    p = synth.layerwise_rows(T=256)
    assert np.array_equal(fused(p), fused(p))


def test_zero_row_and_closed_form():
    # a zero row with eps > 0 stays zero; k equal nonzeros with eps = 0 give
    # gamma * sign * sqrt(W/k) bit-exactly in bf16
    wq, wk, T = 4096, 1024, 3
    x = np.zeros((T, wq + wk))
    for t, (kq, kk) in enumerate([(0, 0), (4, 1), (16, 4)]):
        if kq:
            x[t, np.arange(0, wq, wq // kq)[:kq]] = -2.5
            x[t, wq + np.arange(0, wk, wk // kk)[:kk]] = 0.625
    p = synth.Problem("closed", synth.BF16, T, wq + wk, wq, wk, synth.to_dtype(x, synth.BF16),
                      synth.make_gamma(9, 3, wq, synth.BF16), synth.make_gamma(9, 4, wk, synth.BF16),
                      0.0, nshards=8)
    got = fused(p)
    gq = oracle.decode(p.gamma_q, synth.BF16)
    gk = oracle.decode(p.gamma_k, synth.BF16)
    want = np.zeros_like(x)
    for t, (kq, kk) in enumerate([(0, 0), (4, 1), (16, 4)]):
        if kq:
            iq = np.arange(0, wq, wq // kq)[:kq]
            ik = np.arange(0, wk, wk // kk)[:kk]
            want[t, iq] = -gq[iq] * np.sqrt(wq / kq)
            want[t, wq + ik] = gk[ik] * np.sqrt(wk / kk)
    assert np.array_equal(got[1:], synth.to_dtype(want, synth.BF16)[1:]), "closed form rows"
    assert np.all(np.isnan(oracle.decode(got[0], synth.BF16))), "0/sqrt(0) is NaN with eps = 0"
    p.eps = synth.eps_f32(1e-6)
    got = fused(p)
    assert np.all(oracle.decode(got[0], synth.BF16) == 0.0)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F8], ids=["bf16", "fp8"])
def test_graph_replay_matches_eager(dtype):
    """The fused call, and partial_sumsq followed by apply_scalar, captured in
    graphs: every replay (with eager work and synchronisations between them)
    leaves the bytes the eager calls leave, and the partials too."""
    p = synth.layerwise_problem(f"graph_{synth.DTYPE_NAMES[dtype]}", 61, dtype, 96, 4096, 1024, 6144, 8,
                                outlier_frac=0.01)
    print(f"[layerwise graph] {p.name} T={p.T} R={p.nshards}", flush=True)
    src = host_to_device(p.x, p.dtype)
    gq, gk = _gammas(p)
    R, T = p.nshards, p.T
    pq = torch.empty(R, T, dtype=torch.float32, device="cuda")
    pk = torch.empty(R, T, dtype=torch.float32, device="cuda")

    def fused_call(t):
        q.qknorm_layerwise(t, p.wq, p.wk, gq, gk, p.eps, R)

    def two_phase_call(t):
        q.qknorm_partial_sumsq(t, p.wq, p.wk, R, pq, pk)
        q.qknorm_apply_scalar(t, p.wq, p.wk, pq, pk, p.wq, p.wk, gq, gk, p.eps)

    for name, call in (("fused", fused_call), ("two-phase", two_phase_call)):
        work = src.clone()
        call(work)
        torch.cuda.synchronize()
        eager, eager_pq, eager_pk = work.clone(), pq.clone(), pk.clone()
        work.copy_(src)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                call(work)
        torch.cuda.synchronize()
        for i in range(4):
            work.copy_(src)
            pq.fill_(-1.0)
            pk.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(work.view(torch.uint8), eager.view(torch.uint8)), f"{name}: replay {i}"
            if name == "two-phase":
                assert torch.equal(pq, eager_pq) and torch.equal(pk, eager_pk), f"{name}: partials, replay {i}"
        got = device_to_host(work, p.dtype)
        check_against_oracle(p, got, f"{p.name} {name} graph")
