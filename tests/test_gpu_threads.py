"""Calls from several host threads, each on its own stream with its own
buffers: the library keeps no mutable state between calls (the compute-unit
count it caches per device is written atomically), so every thread's result
is the bytes a single-threaded call gives."""
import threading

import pytest
import torch

import qk_norm_amd as q
from qk_norm_amd import synth
from gpu_util import gamma_to_device, host_to_device

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 12


def _problems():
    ph = synth.fused_gqa_rows(T=96)
    lw = synth.layerwise_rows(T=80)
    return ph, lw


def _per_head(t, p, gq, gk):
    q.qknorm_per_head(t, p.hq, p.hkv, p.head_dim, gq, gk, p.eps)


def _layerwise(t, p, gq, gk):
    q.qknorm_layerwise(t, p.wq, p.wk, gq, gk, p.eps, p.nshards)


def _two_phase(t, p, gq, gk, pq, pk):
    q.qknorm_partial_sumsq(t, p.wq, p.wk, p.nshards, pq, pk)
    q.qknorm_apply_scalar(t, p.wq, p.wk, pq, pk, p.wq, p.wk, gq, gk, p.eps)


def test_concurrent_threads_on_own_streams():
    ph, lw = _problems()
    print(f"[threads] {THREADS} threads x {ROUNDS} rounds: {ph.name}, {lw.name}", flush=True)
    ph_src, lw_src = host_to_device(ph.x, ph.dtype), host_to_device(lw.x, lw.dtype)
    ph_g = (gamma_to_device(ph.gamma_q, ph.dtype), gamma_to_device(ph.gamma_k, ph.dtype))
    lw_g = (gamma_to_device(lw.gamma_q, lw.dtype), gamma_to_device(lw.gamma_k, lw.dtype))

    # single-threaded references on the default stream
    ref_ph = ph_src.clone()
    _per_head(ref_ph, ph, *ph_g)
    ref_lw = lw_src.clone()
    _layerwise(ref_lw, lw, *lw_g)
    torch.cuda.synchronize()

    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()            # default priority
            with torch.cuda.stream(s):
                a, b, c = ph_src.clone(), lw_src.clone(), lw_src.clone()
                pq = torch.empty(lw.nshards, lw.T, dtype=torch.float32, device="cuda")
                pk = torch.empty(lw.nshards, lw.T, dtype=torch.float32, device="cuda")
                for r in range(ROUNDS):
                    a.copy_(ph_src)
                    b.copy_(lw_src)
                    c.copy_(lw_src)
                    _per_head(a, ph, *ph_g)
                    _layerwise(b, lw, *lw_g)
                    _two_phase(c, lw, *lw_g, pq, pk)
                    s.synchronize()
                    for name, got, ref in (("per-head", a, ref_ph), ("layerwise", b, ref_lw),
                                           ("two-phase", c, ref_lw)):
                        if not torch.equal(got.view(torch.int16), ref.view(torch.int16)):
                            errors.append(f"thread {k} round {r}: {name} differs")
        except Exception as e:                  # reported below, in the test's own thread
            errors.append(f"thread {k}: {e!r}")

    ts = [threading.Thread(target=worker, args=(k,)) for k in range(THREADS)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=90)
    assert not any(t.is_alive() for t in ts), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, "; ".join(errors[:5])
