"""QK-Norm bench on one MI355X.

Default workload (the headline metric): per-head QK-Norm, standalone
[T=4096, H=48, D=128] bf16, in place.  One step = one qknorm_per_head call over
one such batch; the batches rotate through a pool of >= 1 GiB of identical
copies so that no step finds its rows in the 256 MB Infinity Cache.

Reported (one JSON line):
  value          whole-job throughput, algorithmic GB/s (each Q/K element read
                 once and written once, plus gamma once) over the timed steps
  ms_per_step    host wall time per step between synchronisations
  roofline       mean launch duration from one HIP event pair around the
                 timed region on the launch stream, algorithmic bytes / that time,
                 against MI355X's 8 TB/s HBM peak; traffic from the committed
                 rocprofv3 counter summary when it matches the current source
  cpu_baseline   the fp64 CPU oracle on the same input, on the host's cores
  cases          the T=32768 large-prefill case (layerwise fused, two-phase,
                 per-head), fused GQA T=8192, and decode-size launch floors

Every bandwidth and projection case first keeps the GPU busy for 0.1 s of
untimed launches (clock warm-up after idle), then runs its W warm-up steps,
then times its K steps.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK-Norm µs/call + achieved HBM GB/s (% of peak), 4096 tok×48 heads×128 bf16"
HBM_PEAK_GBS = 8000.0
POOL_BYTES = 1 << 30
PMC_SUMMARY = os.path.join(ROOT, "profiles", "per_head_bf16_T4096_H48_D128.pmc.md")
# the per-head kernel's code and launch configuration
KERNEL_SOURCES = [os.path.join(ROOT, "qk_norm_amd", "csrc", f) for f in
                  ("qknorm_kernels.hip", "qknorm_device.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(bytes_alg: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if there is none or it was taken on other kernel sources."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    kv = dict(re.findall(r"^- (\w+): ([^\s]+)", text, flags=re.M))
    try:
        if kv.get("source_sha256") != source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------- devices --

def to_device(a, dtype, torch, dev):
    """numpy storage (float32, 16-bit patterns, E4M3 bytes) -> tensor of dtype on dev."""
    import numpy as np
    from qk_norm_amd import synth
    if dtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if dtype == synth.F8:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).view(torch.float8_e4m3fn).to(dev)
    tdt = torch.float16 if dtype == synth.F16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)


def sizes(p):
    """(activation, gamma) bytes per element of problem p."""
    from qk_norm_amd import synth
    return synth.esize(p.dtype), synth.esize(synth.gamma_dtype(p.dtype))


class Timer:
    """Times `steps` back-to-back launches on the launch stream.

    Host wall time covers exactly the `steps` launches, between two
    synchronisations.  One HIP event pair brackets the launches after the
    first LEAD of them: when the first event is stamped the GPU is already
    running the lead launches, and the host stays ahead of the GPU from then
    on, so the bracket holds back-to-back kernels only (no host submission
    time of the first launch); the mean launch duration is its elapsed time
    over the launches it holds.  A separate, shorter pass with an event pair
    around every launch gives the spread (p10/p50/p90); those per-launch
    figures include the events' own overhead (about 2 us each on this part)
    and are reported only as spread.
    """

    LEAD = 2

    def __init__(self, torch):
        self.torch = torch

    def run(self, steps, launch, first=0):
        torch = self.torch
        lead = self.LEAD if steps > self.LEAD else 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if lead == 0:
            e0.record()
        for k, i in enumerate(range(first, first + steps)):
            launch(i)
            if k + 1 == lead:
                e0.record()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1) * 1e3 / (steps - lead)

    def spread(self, steps, launch, first=0):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for k, i in enumerate(range(first, first + steps)):
            ev[k][0].record()
            launch(i)
            ev[k][1].record()
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        n = len(per)
        return {"p10_us": per[int(0.1 * (n - 1))], "p50_us": per[(n - 1) // 2],
                "p90_us": per[int(0.9 * (n - 1))]}


# After an idle spell MI355X runs this kernel about 3 % slower for the first
# ~10 ms of continuous work (measured: 17.0-17.4 us per launch, settling at
# 16.5-16.6 us).  Every bandwidth and projection case therefore keeps the GPU
# busy with untimed launches for CLOCK_WARM_S of wall time before its W
# warm-up steps and K timed steps.  (The decode case measures single-launch
# latency with fixed call counts and has no such phase.)
CLOCK_WARM_S = 0.1


def warm_clocks(torch, launch, first=0, seconds=CLOCK_WARM_S) -> int:
    """Untimed launches for `seconds` of wall time; returns the launch count."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = first
    while time.perf_counter() - t0 < seconds:
        for _ in range(32):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    return i - first


def pool_count(buf_bytes: int, min_copies=2) -> int:
    return max(min_copies, math.ceil(POOL_BYTES / buf_bytes))


# ------------------------------------------------------------------- cases --

def graph_replay_us(torch, launch, steps, first=0):
    """Mean GPU time per launch of `steps` launches captured in one hipGraph and
    replayed (no host work between the launches).  The graph is replayed once
    untimed, then once between a HIP event pair."""
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(first, first + steps):
                launch(i, side.cuda_stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del graph
    return us


def bench_per_head(q, torch, dev, p, steps, warmup, label, max_copies=None, spread=True, graph=False):
    from qk_norm_amd import synth
    lib = q.load()
    es, ges = sizes(p)
    n = pool_count(p.T * p.ld * es)
    if max_copies is not None:
        n = min(n, max_copies)
    base = to_device(p.x, p.dtype, torch, dev)
    pool = [base.clone() for _ in range(n)]
    del base
    gd = synth.gamma_dtype(p.dtype)
    gq = to_device(p.gamma_q, gd, torch, dev)
    gk = to_device(p.gamma_k, gd, torch, dev) if p.gamma_k is not None else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [(t.data_ptr(), p.T, p.ld, p.hq, p.hkv, p.head_dim, gq.data_ptr(),
             gk.data_ptr() if gk is not None else None, p.eps, p.dtype, stream) for t in pool]

    def launch(i):
        rc = lib.qknorm_per_head(*args[i % n])
        if rc:
            raise RuntimeError(f"qknorm_per_head: {q.strerror(rc)}")

    def launch_on(i, s):
        a = args[i % n]
        rc = lib.qknorm_per_head(*a[:-1], s)
        if rc:
            raise RuntimeError(f"qknorm_per_head: {q.strerror(rc)}")

    warm = warm_clocks(torch, launch)
    for i in range(warmup):
        launch(i)
    timer = Timer(torch)
    wall, mean_us = timer.run(steps, launch, first=warmup)
    spread = timer.spread(min(steps, 200), launch, first=warmup + steps) if spread else {}
    if graph:
        spread["graph_replay_us"] = graph_replay_us(torch, launch_on, steps)
    bytes_alg = 2 * p.T * (p.wq + p.wk) * es + (p.head_dim * ges) * (1 + (p.hkv > 0))
    del pool
    torch.cuda.empty_cache()
    log(f"{label}: {mean_us:.2f} us/launch, {bytes_alg / mean_us / 1e3:.0f} GB/s")
    return {"label": label, "bytes": bytes_alg, "wall_s": wall, "steps": steps, "pool": n,
            "clock_warm_launches": warm, "mean_us": mean_us, **spread,
            "gbs": bytes_alg / (mean_us * 1e-6) / 1e9}


def bench_layerwise(q, torch, dev, p, steps, warmup, label="prefill"):
    from qk_norm_amd import synth
    lib = q.load()
    es, ges = sizes(p)
    n = pool_count(p.T * p.ld * es)
    base = to_device(p.x, p.dtype, torch, dev)
    pool = [base.clone() for _ in range(n)]
    del base
    gq = to_device(p.gamma_q, synth.gamma_dtype(p.dtype), torch, dev)
    gk = to_device(p.gamma_k, synth.gamma_dtype(p.dtype), torch, dev)
    pq = torch.empty(p.nshards, p.T, dtype=torch.float32, device=dev)
    pk = torch.empty(p.nshards, p.T, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    R = p.nshards

    def fused(i):
        t = pool[i % n]
        rc = lib.qknorm_layerwise(t.data_ptr(), p.T, p.ld, p.wq, p.wk, gq.data_ptr(), gk.data_ptr(),
                                  p.eps, R, p.dtype, stream)
        if rc:
            raise RuntimeError(q.strerror(rc))

    def partial(i):
        t = pool[i % n]
        rc = lib.qknorm_partial_sumsq(t.data_ptr(), p.T, p.ld, p.wq, p.wk, R, pq.data_ptr(),
                                      pk.data_ptr(), p.dtype, stream)
        if rc:
            raise RuntimeError(q.strerror(rc))

    def apply(i):
        t = pool[i % n]
        rc = lib.qknorm_apply_scalar(t.data_ptr(), p.T, p.ld, p.wq, p.wk, pq.data_ptr(),
                                     pk.data_ptr(), R, p.wq, p.wk, gq.data_ptr(), gk.data_ptr(),
                                     p.eps, p.dtype, stream)
        if rc:
            raise RuntimeError(q.strerror(rc))

    qk_bytes = p.T * (p.wq + p.wk) * es
    g_bytes = (p.wq + p.wk) * ges
    out = {}
    for name, fn, nbytes in (("layerwise_fused", fused, 2 * qk_bytes + g_bytes),
                             ("partial_sumsq", partial, qk_bytes + 2 * R * p.T * 4),
                             ("apply_scalar", apply, 2 * qk_bytes + g_bytes + 2 * R * p.T * 4)):
        warm_clocks(torch, fn)
        for i in range(warmup):
            fn(i)
        wall, mean_us = Timer(torch).run(steps, fn, first=warmup)
        out[name] = {"bytes": nbytes, "mean_us": mean_us, "gbs": nbytes / (mean_us * 1e-6) / 1e9}
        log(f"{label} {name}: {mean_us:.2f} us/launch, {out[name]['gbs']:.0f} GB/s")
    two = out["partial_sumsq"]["mean_us"] + out["apply_scalar"]["mean_us"]
    out["two_phase_total"] = {"mean_us": two, "bytes": 3 * qk_bytes + g_bytes + 4 * R * p.T * 4,
                              "gbs_vs_fused_alg_bytes": (2 * qk_bytes + g_bytes) / (two * 1e-6) / 1e9}
    del pool
    torch.cuda.empty_cache()
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0

# The pages' own figures, on other hardware: context for the bench line, not
# targets (the dtype of the per-head tables is not stated on the pages).
PAGES_CONTEXT = {
    "kind": "the pages' numbers on other hardware; context only, not a target",
    "per_head_T4096_H48_D128_us": {
        "source": "sglang PR 13189 (turbomind_rms_norm for QK norm), benchmark tables",
        "H20": {"sglang_rmsnorm": 269.633, "turbomind_rms_norm": 69.378},
        "H100": {"sglang_rmsnorm": 271.742, "turbomind_rms_norm": 73.303},
    },
    "layerwise_qknorm_latency_reduction_pct": {
        "source": "SwiftQK (arXiv 2608.09160), abstract",
        "range": [81.4, 93.9],
        "setting": "multi-GPU tensor parallel: scalar sum-of-squares exchange against a full-vector "
                   "all-gather; there is no single-GPU figure",
    },
}


def bench_proj(q, torch, dev, steps, warmup, T=4096, hidden=4096, hq=32, hkv=8, D=128, copies=1):
    """QKV projection of a Qwen3-8B-sized layer ([T, 4096] x [6144, 4096]^T,
    32 Q + 8 K + 8 V heads of 128): fused with per-head QK-Norm, the plain
    projection (same kernel), torch's mm (hipBLASLt), and mm + qknorm_per_head;
    at decode sizes also the fused projection through a workspace.  x and w
    stay resident; with copies > 1 the calls rotate through that many copies
    of the 48 MB weight, so that the 256 MB Infinity Cache cannot hold it from
    one call to the next (in a served model the other layers' weights come
    between two calls of one layer)."""
    import numpy as np
    from qk_norm_amd import synth
    N = (hq + 2 * hkv) * D
    x = to_device(synth.make_x(90, T, hidden, synth.BF16, token_scale=(0.25, 4.0)), synth.BF16, torch, dev)
    w0 = to_device(synth.to_dtype(synth.normal(91, 0, N * hidden).reshape(N, hidden) / np.sqrt(hidden),
                                  synth.BF16), synth.BF16, torch, dev)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    gq = to_device(synth.make_gamma(90, 3, D, synth.BF16), synth.BF16, torch, dev)
    gk = to_device(synth.make_gamma(90, 4, D, synth.BF16), synth.BF16, torch, dev)
    out = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    out2 = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    lib = q.load()
    stream = torch.cuda.current_stream(dev).cuda_stream

    need = q.qknorm_qkv_proj_workspace_bytes(T, hq, hkv, D)
    space = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    wptr = [t.data_ptr() for t in ws]

    def proj(flags):
        def f(i):
            rc = lib.qknorm_qkv_proj_per_head(x.data_ptr(), hidden, wptr[i % copies], hidden, out.data_ptr(),
                                              N, T, hidden, hq, hkv, D, gq.data_ptr(), gk.data_ptr(),
                                              1e-6, flags, synth.BF16, stream)
            if rc:
                raise RuntimeError(q.strerror(rc))
        return f

    def proj_ws(i):
        rc = lib.qknorm_qkv_proj_per_head_ws(x.data_ptr(), hidden, wptr[i % copies], hidden, out.data_ptr(),
                                             N, T, hidden, hq, hkv, D, gq.data_ptr(), gk.data_ptr(),
                                             1e-6, 0, synth.BF16, space.data_ptr(), need, stream)
        if rc:
            raise RuntimeError(q.strerror(rc))

    def mm(i):
        torch.mm(x, ws[i % copies].t(), out=out2)

    def mm_norm(i):
        torch.mm(x, ws[i % copies].t(), out=out2)
        rc = lib.qknorm_per_head(out2.data_ptr(), T, N, hq, hkv, D, gq.data_ptr(), gk.data_ptr(), 1e-6,
                                 synth.BF16, stream)
        if rc:
            raise RuntimeError(q.strerror(rc))

    flops = 2.0 * T * hidden * N
    res = {"shape": {"T": T, "hidden": hidden, "N": N, "hq": hq, "hkv": hkv, "head_dim": D},
           "flops": flops, "weight_copies": copies}
    variants = (("fused_proj_qknorm", proj(0)), ("plain_proj", proj(1)),
                ("torch_mm", mm), ("torch_mm_then_qknorm", mm_norm))
    if need:
        variants += (("fused_proj_qknorm_ws", proj_ws),)
    # compute-bound kernels: warm every variant first (clocks), then take the
    # better of two timed rounds of each
    for _, fn in variants:
        warm_clocks(torch, fn)
        for i in range(warmup):
            fn(i)
    best = {}
    for _ in range(2):
        for name, fn in variants:
            _, us = Timer(torch).run(steps, fn, first=warmup)
            best[name] = min(us, best.get(name, us))
    for name, _ in variants:
        us = best[name]
        res[name] = {"mean_us": us, "tflops": flops / (us * 1e-6) / 1e12,
                     "frac_of_mfma_peak": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        log(f"proj T={T} {name}: {us:.1f} us, {res[name]['tflops']:.0f} TFLOP/s")
    del x, w0, ws, out, out2, space
    torch.cuda.empty_cache()
    return res


def bench_decode(q, torch, dev, reps=200):
    """Decode-sized launches: per-head [T, 48, 128] bf16 for T in {1, 8, 16, 64, 128}
    and layerwise [T, 6144] (Q 4096 + K 1024, 8 shards) for T in {1, 4, 32, 256}.
    For each: host time per eager call through the binding, GPU time per launch
    from one event pair around `reps` back-to-back launches, and per launch in a
    replayed hipGraph of `reps` launches."""
    from qk_norm_amd import synth
    out = []

    def measure(launch):
        for _ in range(20):
            launch()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            launch()
        host_us = (time.perf_counter() - t0) / reps * 1e6
        torch.cuda.synchronize()
        _, gpu_us = Timer(torch).run(reps, lambda _i: launch())
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for _ in range(reps):
                    launch()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return host_us, gpu_us, e0.elapsed_time(e1) * 1e3 / reps

    for T in (1, 8, 16, 64, 128):
        p = synth.standalone_heads(T=T, H=48)
        x = to_device(p.x, p.dtype, torch, dev)
        g = to_device(p.gamma_q, p.dtype, torch, dev)
        h, gpu, gr = measure(lambda: q.qknorm_per_head(x, 48, 0, 128, g, None, p.eps))
        out.append({"mode": "per_head", "T": T, "H": 48, "host_us_per_eager_call": h,
                    "gpu_us_per_launch_back_to_back": gpu, "graph_us_per_launch": gr})
        log(f"decode per-head T={T}: host {h:.2f} us, back-to-back {gpu:.2f} us, graph {gr:.2f} us")
    for T in (1, 4, 32, 256):
        p = synth.layerwise_rows(T=T)
        x = to_device(p.x, p.dtype, torch, dev)
        gq = to_device(p.gamma_q, p.dtype, torch, dev)
        gk = to_device(p.gamma_k, p.dtype, torch, dev)
        h, gpu, gr = measure(lambda: q.qknorm_layerwise(x, p.wq, p.wk, gq, gk, p.eps, p.nshards))
        out.append({"mode": "layerwise", "T": T, "wq": p.wq, "wk": p.wk, "nshards": p.nshards,
                    "host_us_per_eager_call": h, "gpu_us_per_launch_back_to_back": gpu,
                    "graph_us_per_launch": gr})
        log(f"decode layerwise T={T}: host {h:.2f} us, back-to-back {gpu:.2f} us, graph {gr:.2f} us")
    return out


# The grid of the sglang PR's per-head tables (head_dim 128), and its
# turbomind_rms_norm column in us per call, as context (dtype not stated).
PR_GRID_T = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)
PR_TURBOMIND_US = {
    "H20": {16: (2.401, 2.554, 2.554, 2.606, 2.623, 2.670, 2.768, 2.878, 3.171, 4.080, 5.538, 8.726, 15.672),
            32: (2.553, 2.554, 2.609, 2.623, 2.670, 2.768, 2.862, 3.171, 4.080, 5.537, 8.731, 15.645, 44.130),
            48: (2.548, 2.591, 2.612, 2.651, 2.723, 2.813, 3.288, 3.487, 4.873, 7.115, 11.958, 28.149, 69.378)},
    "H100": {16: (2.644, 2.749, 2.758, 2.785, 2.903, 3.018, 3.067, 3.305, 3.481, 4.106, 5.459, 8.214, 16.025),
             32: (2.760, 2.737, 2.813, 2.903, 3.021, 3.063, 3.286, 3.476, 4.112, 5.469, 8.206, 16.015, 46.956),
             48: (2.732, 2.763, 2.831, 2.940, 2.998, 3.143, 3.355, 3.842, 4.792, 6.965, 11.216, 29.693, 73.303)},
}


def _graph_and_eager(torch, dev, launch, reps):
    """GPU time per launch of `reps` eager launches (event pair, after the
    clock warm-up) and of `reps` launches replayed from one captured hipGraph.
    `launch(j, stream)` launches call j on the given raw stream."""
    cur = torch.cuda.current_stream(dev).cuda_stream
    warm_clocks(torch, lambda j: launch(j, cur))
    _, eager_us = Timer(torch).run(reps, lambda j: launch(j, cur))
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for j in range(reps):
                launch(j, side.cuda_stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / reps
    del graph
    return graph_us, eager_us


def _per_head_points(q, torch, dev, problems, reps, label):
    """Graph-replay and eager time per launch for each per-head problem, its
    buffers rotating through up to 64 copies (so the smaller sizes run out of
    the caches, as a serving loop's would)."""
    from qk_norm_amd import synth
    lib = q.load()
    out = []
    for p in problems:
        es, ges = sizes(p)
        n = min(pool_count(p.T * p.ld * es), 64)
        base = to_device(p.x, p.dtype, torch, dev)
        pool = [base.clone() for _ in range(n)]
        gq = to_device(p.gamma_q, synth.gamma_dtype(p.dtype), torch, dev)
        gk = to_device(p.gamma_k, synth.gamma_dtype(p.dtype), torch, dev) if p.hkv else None
        bytes_alg = 2 * p.T * (p.wq + p.wk) * es + p.head_dim * ges * (2 if p.hkv else 1)

        def launch(j, stream):
            rc = lib.qknorm_per_head(pool[j % n].data_ptr(), p.T, p.ld, p.hq, p.hkv, p.head_dim,
                                     gq.data_ptr(), gk.data_ptr() if gk is not None else None, p.eps,
                                     p.dtype, stream)
            if rc:
                raise RuntimeError(q.strerror(rc))

        graph_us, eager_us = _graph_and_eager(torch, dev, launch, reps)
        gbs = bytes_alg / (graph_us * 1e-6) / 1e9
        out.append({"hq": p.hq, "hkv": p.hkv, "T": p.T, "ld": p.ld, "graph_us": graph_us,
                    "eager_us": eager_us, "gbs_graph": gbs, "pct_of_hbm_peak_graph": 100 * gbs / HBM_PEAK_GBS,
                    "pool": n})
        log(f"{label} hq={p.hq} hkv={p.hkv} T={p.T}: graph {graph_us:.2f} us, eager {eager_us:.2f} us")
        del pool, base
        torch.cuda.empty_cache()
    return out


def bench_sweep(q, torch, dev, reps=200):
    """Per-head bf16 [T, H, 128] over the PR's grid (H in {16, 32, 48}, T = 1 ... 4096).
    For each point: GPU time per launch of `reps` launches replayed from one
    captured hipGraph (no host cost between launches), and of `reps` eager
    launches through the C ABI (host-bound at small T)."""
    from qk_norm_amd import synth
    out = []
    for H in (16, 32, 48):
        pts = _per_head_points(q, torch, dev, [synth.standalone_heads(T=T, H=H) for T in PR_GRID_T], reps,
                               "sweep")
        for i, r in enumerate(pts):
            out.append({"H": H, "T": r["T"], "graph_us": r["graph_us"], "eager_us": r["eager_us"],
                        "gbs_graph": r["gbs_graph"], "pct_of_hbm_peak_graph": r["pct_of_hbm_peak_graph"],
                        "pool": r["pool"], "pages_turbomind_us": {k: v[H][i] for k, v in PR_TURBOMIND_US.items()}})
    return out


def bench_gqa_sweep(q, torch, dev, reps=200):
    """Per-head on fused GQA rows [T, 6144] (Q 32 + K 8 heads of 128, V 8 heads
    untouched), bf16, T in {1, 8, 64, 512, 8192}: the same two timings."""
    from qk_norm_amd import synth
    return _per_head_points(q, torch, dev, [synth.fused_gqa_rows(T=T) for T in (1, 8, 64, 512, 8192)], reps,
                            "fused GQA")


def bench_d2d_copy(torch, dev, nbytes, steps=400, warmup=40):
    """A device-to-device copy (hipMemcpyAsync through torch's copy_) that reads and
    writes as many bytes as one headline launch: the practical ceiling the
    runtime's own copy reaches.  Buffer pairs rotate through >= 1 GiB."""
    n = pool_count(2 * nbytes)
    src = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(n)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(n)]

    def launch(i):
        dst[i % n].copy_(src[i % n])

    warm_clocks(torch, launch)
    for i in range(warmup):
        launch(i)
    _, mean_us = Timer(torch).run(steps, launch, first=warmup)
    del src, dst
    torch.cuda.empty_cache()
    log(f"d2d copy of {nbytes} bytes: {mean_us:.2f} us, {2 * nbytes / mean_us / 1e3:.0f} GB/s")
    return {"bytes_read": nbytes, "bytes_written": nbytes, "mean_us": mean_us,
            "gbs": 2 * nbytes / (mean_us * 1e-6) / 1e9}


CEILING_LIB = os.path.join(ROOT, "qk_norm_amd", "libqknorm_ceiling.so")
STREAM_MODES = {0: "in_place", 1: "read_only", 2: "write_only"}
# (vectors per lane per trip, threads per block, grid cap in blocks per CU; 0 = one trip)
STREAM_SHAPES = ((1, 256, 0), (2, 256, 0), (1, 512, 0), (2, 512, 0), (4, 512, 0),
                 (1, 256, 16), (1, 256, 24), (2, 256, 8), (2, 256, 12), (2, 256, 16),
                 (1, 512, 8), (1, 512, 12), (2, 512, 4), (2, 512, 6), (2, 512, 8),
                 (1, 1024, 0), (2, 1024, 0))


def bench_stream(torch, dev, nbytes, steps=200, warmup=20, modes=(0, 1, 2)):
    """Trivial streams over `nbytes` per launch with the norms' access width and
    cache policy (16-byte buffer loads/stores, nt sc1): in place (read and write
    every byte once), read only, write only; each over STREAM_SHAPES, buffers
    rotating through >= 1 GiB.  The fastest shape of each mode is the practical
    ceiling for a kernel that moves those bytes."""
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(CEILING_LIB)
    lib.qknorm_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.qknorm_ceiling_stream.restype = ctypes.c_int32
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n = pool_count(nbytes)
    pool = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = {"bytes_per_direction": nbytes, "pool": n}
    for mode in modes:
        moved = nbytes * (2 if mode == 0 else 1)
        rows = []
        for u, threads, cap in STREAM_SHAPES:
            max_blocks = cus * cap

            def launch(i, u=u, threads=threads, max_blocks=max_blocks):
                rc = lib.qknorm_ceiling_stream(pool[i % n].data_ptr(), nbytes, mode, u, threads, max_blocks,
                                               sink.data_ptr(), stream)
                if rc:
                    raise RuntimeError(f"ceiling probe rc={rc}")

            warm_clocks(torch, launch)
            for i in range(warmup):
                launch(i)
            _, us = Timer(torch).run(steps, launch, first=warmup)
            rows.append({"u": u, "threads": threads, "blocks_per_cu_cap": cap, "mean_us": us,
                         "gbs": moved / (us * 1e-6) / 1e9})
        best = min(rows, key=lambda r: r["mean_us"])
        out[STREAM_MODES[mode]] = {"best": best, "bytes_moved": moved, "shapes": rows}
        log(f"stream {STREAM_MODES[mode]} {nbytes / 2**20:.0f} MiB: best {best['mean_us']:.2f} us "
            f"({best['gbs']:.0f} GB/s) at u={best['u']} threads={best['threads']} cap={best['blocks_per_cu_cap']}")
    del pool
    torch.cuda.empty_cache()
    return out


def summarize_trace(path, kernel, skip=0, count=0, nbytes=0.0, workgroup=0, grid=0):
    """Kernel-trace CSV of rocprofv3 -> durations of the dispatches of kernels
    whose name contains `kernel` (and, if given, of that workgroup and grid size
    in threads along x), in dispatch order: the window [skip, skip+count)
    (count 0: to the end).  Returns a dict of statistics in us."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if workgroup and int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 0) != workgroup:
                continue
            if grid and int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0) != grid:
                continue
            if kernel in r["Kernel_Name"]:
                rows.append((int(r.get("Dispatch_Id") or 0), int(r["Start_Timestamp"]),
                             int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort(key=lambda r: (r[1], r[0]))
    total = len(rows)
    win = rows[skip:skip + count] if count else rows[skip:]
    if not win:
        raise SystemExit(f"no dispatches of {kernel!r} in the window (found {total})")
    d = sorted((e - b) / 1e3 for _, b, e, _ in win)
    m = len(d)
    avg = sum(d) / m
    name = win[0][3]
    name = name[:name.index(">(") + 1] if ">(" in name else name.split("(")[0]
    res = {"kernel": name, "dispatches_of_kernel": total, "window": [skip, skip + m],
           "launches": m, "avg_us": avg, "p10_us": d[int(0.1 * (m - 1))], "median_us": d[(m - 1) // 2],
           "p90_us": d[int(0.9 * (m - 1))], "min_us": d[0], "max_us": d[-1]}
    if nbytes:
        res["gbs_at_avg"] = nbytes / (avg * 1e-6) / 1e9
        res["pct_of_8tbs"] = 100 * res["gbs_at_avg"] / HBM_PEAK_GBS
    return res


def oracle_threads_all() -> tuple[int, int]:
    """(threads for the all-cores leg, host CPUs visible to this process).
    The all-cores leg uses every CPU in the affinity mask, capped by
    OMP_NUM_THREADS when the environment sets it (a host shared between jobs
    gives each job that many)."""
    visible = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    except ValueError:
        cap = 0
    return (min(visible, cap) if cap > 0 else visible), visible


def cpu_baseline(p, q, torch, dev, run_s=2.0):
    """The fp64 C oracle on the headline input, at 1 thread and on all host
    cores: three runs per leg of about run_s seconds each (whole calls), the
    median run's time per call reported.  The oracle's first result also
    checks one fresh GPU launch on the same input, element by element (the
    tolerance the tests use for bf16)."""
    import numpy as np
    import oracle
    bytes_alg = 2 * p.T * (p.wq + p.wk) * 2 + p.head_dim * 2
    all_threads, visible = oracle_threads_all()
    ref = None
    legs = {}
    for leg, want in (("one_thread", 1), ("all_cores", all_threads)):
        used = oracle.set_threads(want)
        runs, calls = [], []
        for _ in range(3):
            n, t0 = 0, time.perf_counter()
            while True:
                r = oracle.per_head(p.x, p.dtype, p.hq, p.hkv, p.head_dim, p.gamma_q, p.gamma_k, p.eps,
                                    want_y=ref is None)
                ref = ref or r
                n += 1
                el = time.perf_counter() - t0
                if el >= run_s:
                    break
            runs.append(el / n)
            calls.append(n)
        med = sorted(runs)[1]
        legs[leg] = {"threads": used, "us_per_call_median_of_3": med * 1e6,
                     "us_per_call_runs": [r * 1e6 for r in runs], "calls_per_run": calls,
                     "gbs": bytes_alg / med / 1e9}
    oracle.set_threads(all_threads)
    # one launch on a fresh copy of the same input
    x = to_device(p.x, p.dtype, torch, dev)
    q.qknorm_per_head(x, p.hq, p.hkv, p.head_dim, to_device(p.gamma_q, p.dtype, torch, dev),
                      None, p.eps)
    torch.cuda.synchronize()
    got = x.cpu().view(torch.int16).numpy().view(np.uint16)
    y64, yr = ref
    g = oracle.decode(got, p.dtype)
    nz = y64 != 0
    rel = np.abs(g[nz] - y64[nz]) / np.abs(y64[nz])

    def ordinal(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)

    ulp = np.abs(ordinal(got) - ordinal(yr))
    parity = {"elements": int(got.size), "max_rel_err": float(rel.max()),
              "rtol": 8e-3, "zero_where_oracle_zero": bool(np.all(g[~nz] == 0)),
              "ulp_0": int((ulp == 0).sum()), "ulp_1": int((ulp == 1).sum()),
              "ulp_over_1": int((ulp > 1).sum())}
    parity["pass"] = bool(parity["max_rel_err"] <= 8e-3 and parity["zero_where_oracle_zero"]
                          and parity["ulp_over_1"] == 0)
    a, o = legs["all_cores"], legs["one_thread"]
    return {"value": a["gbs"], "unit": "GB/s", "cores": a["threads"], "kind": "oracle",
            "sample": f"whole calls of the fp64 C oracle on the same [4096,48,128] bf16 input, "
                      f"3 runs of >= {run_s:.0f} s per leg, median run; all-cores leg "
                      f"{a['threads']} threads ({visible} host CPUs visible), "
                      f"one-thread leg {o['gbs']:.2f} GB/s",
            "us_per_call": a["us_per_call_median_of_3"], "host_cpus_visible": visible,
            "legs": legs, "parity_of_one_gpu_launch": parity}


# -------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--quick", action="store_true", help="headline case only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--case", default="headline",
                    choices=["headline", "prefill_layerwise", "prefill_per_head", "fp8_per_head",
                             "fp8_prefill_layerwise", "proj", "proj_tokens", "decode", "sweep", "copy", "stream",
                             "wide_layerwise"],
                    help="single case for profiling runs")
    ap.add_argument("--stream-shape", metavar="U,THREADS,CAP",
                    help="with --case stream: one in-place shape only (CAP in blocks per CU, 0: one trip)")
    ap.add_argument("--stream-mib", type=int, default=48, help="with --stream-shape: MiB per direction")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="summarise a rocprofv3 kernel-trace CSV (no GPU use) and exit")
    ap.add_argument("--kernel", default="per_head_kernel", help="with --summarize-trace: name substring")
    ap.add_argument("--skip", type=int, default=0, help="with --summarize-trace: dispatches to skip")
    ap.add_argument("--count", type=int, default=0, help="with --summarize-trace: dispatches to take")
    ap.add_argument("--bytes", type=float, default=0.0, help="with --summarize-trace: bytes per launch")
    ap.add_argument("--workgroup", type=int, default=0, help="with --summarize-trace: workgroup size")
    ap.add_argument("--grid", type=int, default=0, help="with --summarize-trace: grid size in threads")
    args = ap.parse_args()

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.kernel, args.skip, args.count,
                                         args.bytes, args.workgroup, args.grid)))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this QK-Norm build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import qk_norm_amd as q
    from qk_norm_amd import synth
    q.load()
    dev = torch.device("cuda:0")

    if args.case == "copy":
        # plain device copy of known size, for scaling the FETCH/WRITE counters
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"case": "copy", "bytes_read": n, "bytes_written": n}))
        return
    if args.case == "stream":
        res = {"case": "stream"}
        if args.stream_shape:
            # one in-place shape at one size (for a kernel trace of the ceiling)
            u, threads, cap = (int(v) for v in args.stream_shape.split(","))
            global STREAM_SHAPES
            STREAM_SHAPES = ((u, threads, cap),)
            res[f"{args.stream_mib}MiB"] = bench_stream(torch, dev, args.stream_mib << 20, args.steps,
                                                       args.warmup, modes=(0,))
        else:
            for mib in (24, 48, 288, 576):
                res[f"{mib}MiB"] = bench_stream(torch, dev, mib << 20)
        print(json.dumps(res))
        return
    if args.case == "wide_layerwise":
        # rows too wide for the register-resident kernels: Q 32768 + K 4096
        # bf16 columns, 8 shards (the streamed layerwise kernel)
        p = synth.layerwise_problem("wide_layerwise", 71, synth.BF16, 4096, 32768, 4096, 32768 + 2 * 4096,
                                    8, outlier_frac=0.01)
        print(json.dumps({"case": "wide_layerwise", **bench_layerwise(q, torch, dev, p, args.steps,
                                                                      args.warmup, "wide [4096, 40960]")}))
        return
    if args.case == "prefill_layerwise":
        p = synth.prefill_rows(T=32768)
        print(json.dumps({"case": "prefill_layerwise", **bench_layerwise(q, torch, dev, p, args.steps, args.warmup)}))
        return
    if args.case == "fp8_per_head":
        p = synth.standalone_heads(T=4096, H=48, dtype=synth.F8)
        print(json.dumps({"case": "fp8_per_head",
                          **bench_per_head(q, torch, dev, p, args.steps, args.warmup, "fp8 per-head",
                                           graph=True)}))
        return
    if args.case == "fp8_prefill_layerwise":
        p = synth.prefill_rows(T=32768, dtype=synth.F8)
        print(json.dumps({"case": "fp8_prefill_layerwise",
                          **bench_layerwise(q, torch, dev, p, args.steps, args.warmup, "fp8 prefill [32768, 10240]")}))
        return
    if args.case == "sweep":
        from qk_norm_amd import synth
        print(json.dumps({"case": "sweep", "per_head_bf16_D128": bench_sweep(q, torch, dev),
                          "fused_gqa_rows_bf16": bench_gqa_sweep(q, torch, dev),
                          "fused_rows_f32_T4": _per_head_points(q, torch, dev, [synth.small_fused_f32()], 200,
                                                                "fp32 fused rows")}))
        return
    if args.case == "decode":
        print(json.dumps({"case": "decode", "launches": bench_decode(q, torch, dev)}))
        return
    if args.case == "proj":
        print(json.dumps({"case": "proj", **bench_proj(q, torch, dev, args.steps, args.warmup, T=8192)}))
        return
    if args.case == "proj_tokens":
        # the Qwen3-8B projection from decode sizes to prefill (tiles of 64,
        # 128 or 256 rows by token count; up to 64 tokens also the split
        # kernels through a workspace), the weight rotating through 6 copies
        # (300 MB)
        pts = {}
        for T in (1, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096):
            r = bench_proj(q, torch, dev, args.steps, args.warmup, T=T, copies=6)
            pts[str(T)] = {k: round(r[k]["mean_us"], 2) for k in
                           ("fused_proj_qknorm", "fused_proj_qknorm_ws", "plain_proj", "torch_mm",
                            "torch_mm_then_qknorm") if k in r}
        print(json.dumps({"case": "proj_tokens", "weight_copies": 6, "us_per_call": pts}))
        return
    if args.case == "prefill_per_head":
        p = synth.prefill_rows(T=32768, mode="per_head")
        print(json.dumps({"case": "prefill_per_head",
                          **bench_per_head(q, torch, dev, p, args.steps, args.warmup, "prefill [32768, 10240] per-head")}))
        return

    t_start = time.perf_counter()
    p = synth.standalone_heads(T=4096, H=48)
    head = bench_per_head(q, torch, dev, p, args.steps, args.warmup, "headline per-head")
    lead = Timer.LEAD if args.steps > Timer.LEAD else 0
    bytes_alg = head["bytes"]
    value = bytes_alg * args.steps / head["wall_s"] / 1e9
    achieved = head["gbs"]
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["wall_s"] / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "io_dtype": "bf16", "data": "synthetic",
        "config": {"workload": "per-head QK-Norm, standalone [T=4096, H=48, D=128] bf16, in place",
                   "T": 4096, "H": 48, "head_dim": 128, "eps": 1e-6, "seed": p.seed,
                   "rotating_pool_copies": head["pool"],
                   "untimed_clock_warmup": f"{head['clock_warm_launches']} launches "
                                           f"({CLOCK_WARM_S} s) before the W warm-up steps"},
        "us_per_call": round(head["mean_us"], 3),
        "us_per_call_spread_p10_p50_p90_with_event_overhead":
            [round(head["p10_us"], 3), round(head["p50_us"], 3), round(head["p90_us"], 3)],
        "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(bytes_alg),
                     "kernel": "per_head_kernel<bf16, 16 lanes/head>",
                     "bytes_per_launch": bytes_alg,
                     "timing": f"HIP event pair on the launch stream around the last "
                               f"{args.steps - lead} of the {args.steps} timed launches"},
        # where the timed launches sit among this kernel's dispatches in a
        # rocprofv3 kernel trace of this run (for --summarize-trace)
        "trace_window": {"kernel": "per_head_kernel<1, 16, 2, true, true, true, false>",
                         "skip": head["clock_warm_launches"] + args.warmup + lead,
                         "count": args.steps - lead},
    }
    if not args.quick:
        cases = {}
        for mib, kern_us in ((48, head["mean_us"]), (24, None)):
            st = bench_stream(torch, dev, mib << 20, modes=(0,))
            best = st["in_place"]["best"]
            cases[f"stream_ceiling_in_place_{mib}MiB"] = {"best": best, "shapes": st["in_place"]["shapes"]}
            if kern_us is not None:
                result["headline_frac_of_stream_ceiling_48MiB"] = round(best["mean_us"] / kern_us, 4)
        p5 = synth.prefill_rows(T=32768)
        cases["prefill_T32768_layerwise"] = bench_layerwise(q, torch, dev, p5, 50, 5)
        p5h = synth.prefill_rows(T=32768, mode="per_head")
        del p5
        c = bench_per_head(q, torch, dev, p5h, 50, 5, "prefill [32768, 10240] per-head")
        cases["prefill_T32768_per_head"] = {k: c[k] for k in ("bytes", "mean_us", "gbs")}
        del p5h
        c = bench_per_head(q, torch, dev, synth.fused_gqa_rows(T=8192), 100, 10, "fused GQA [8192, 6144] per-head")
        cases["fused_gqa_T8192_per_head"] = {k: c[k] for k in ("bytes", "mean_us", "gbs")}
        for dt in (synth.F16, synth.F8):
            name = synth.DTYPE_NAMES[dt]
            c = bench_per_head(q, torch, dev, synth.standalone_heads(T=4096, H=48, dtype=dt), 400, 40,
                               f"{name} per-head [4096, 48, 128]", graph=dt == synth.F8)
            cases[f"{name}_T4096_H48_per_head"] = {k: c[k] for k in ("bytes", "mean_us", "gbs")}
            if "graph_replay_us" in c:
                cases[f"{name}_T4096_H48_per_head"]["graph_replay_us"] = c["graph_replay_us"]
            if dt == synth.F8:
                ceil_us = cases["stream_ceiling_in_place_24MiB"]["best"]["mean_us"]
                cases[f"{name}_T4096_H48_per_head"]["frac_of_stream_ceiling_24MiB"] = ceil_us / c["mean_us"]
        p8 = synth.prefill_rows(T=32768, dtype=synth.F8)
        cases["fp8e4m3_prefill_T32768_layerwise"] = bench_layerwise(q, torch, dev, p8, 50, 5,
                                                                 "fp8e4m3 [32768, 10240]")
        del p8
        cases["decode"] = bench_decode(q, torch, dev)
        cp = bench_d2d_copy(torch, dev, p.T * (p.wq + p.wk) * 2)
        cases["d2d_copy_headline_bytes"] = {**cp, "copy_time_over_headline_kernel_time": cp["mean_us"] / head["mean_us"]}
        for T in (4096, 8192):
            cases[f"qkv_proj_T{T}_qwen3_8b"] = bench_proj(q, torch, dev, 30, 5, T=T)
        # the weight rotating through 6 copies (300 MB), cold in the Infinity
        # Cache at each call as in a served model; decode sizes add the
        # workspace form
        for T in (1, 16, 4096, 8192):
            cases[f"qkv_proj_T{T}_qwen3_8b_cold_weight"] = bench_proj(q, torch, dev, 30, 5, T=T, copies=6)
        result["cases"] = cases
    result["pages_context"] = PAGES_CONTEXT
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(p, q, torch, dev)
    result["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
