"""The seeded input generator (CPU only)."""
import os

import numpy as np
import pytest

import oracle
from qk_norm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_known_answer():
    # SplitMix64 from state 0: the first three outputs of the published generator.
    i = np.arange(1, 4, dtype=np.uint64)
    z = np.uint64(0) + i * synth._GOLDEN
    synth._mix(z)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_deterministic_and_seed_dependent():
    a = synth.make_x(7, 5, 300, synth.BF16)
    b = synth.make_x(7, 5, 300, synth.BF16)
    c = synth.make_x(8, 5, 300, synth.BF16)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_rows_regenerate_on_their_own():
    full = synth.make_x(3, 40, 1000, synth.BF16, token_scale=(0.1, 10), outlier_frac=0.01)
    part = synth.make_x(3, 7, 1000, synth.BF16, token_scale=(0.1, 10), outlier_frac=0.01,
                        row_start=17)
    assert np.array_equal(full[17:24], part)
    # odd starts split a Box-Muller pair
    n = synth.normal(5, 0, 101)
    assert np.array_equal(n[33:70], synth.normal(5, 0, 37, start=33))


def test_large_threaded_path_matches_small():
    n = synth._CHUNK * 2 + 12345
    big = synth.normal(9, 0, n)
    assert np.array_equal(big[:1000], synth.normal(9, 0, 1000))
    s = synth._CHUNK + 5
    assert np.array_equal(big[s:s + 777], synth.normal(9, 0, 777, start=s))


def test_distributions():
    z = synth.normal(11, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    u = synth.uniform(11, 1, 1 << 20)
    assert u.min() > 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 2e-3
    g = oracle.decode(synth.make_gamma(11, 3, 4096, synth.BF16), synth.BF16)
    assert g.min() >= 0.5 and g.max() <= 1.5


def test_outliers_and_token_scale():
    assert len(synth.outlier_columns(4, 6144, 0.01)) == 61
    assert len(synth.outlier_columns(5, 10240, 0.01)) == 102
    p = synth.layerwise_rows(T=32)
    x = oracle.decode(p.x, synth.BF16)
    cols = synth.outlier_columns(4, 6144, 0.01)
    others = np.setdiff1d(np.arange(6144), cols)
    assert np.abs(x[:, cols]).mean() > 10 * np.abs(x[:, others]).mean()
    p2 = synth.standalone_heads(T=64, H=16)
    rms = np.sqrt(np.mean(oracle.decode(p2.x, synth.BF16) ** 2, axis=1))
    assert rms.min() > 0.05 and rms.max() < 12 and rms.max() / rms.min() > 5


def test_bf16_rounding_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    v = (synth.normal(12, 0, 100000) * 50).astype(np.float32)
    mine = synth.round_bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


def test_fused_gqa_layout_matches_the_lesson():
    g = _golden("gqa_fused_split.txt")
    p = synth.fused_gqa_rows(T=2)
    assert p.hq == g["q_heads"] and p.hkv == g["kv_heads"] and p.head_dim == g["head_dim"]
    assert p.wq == g["q_width"] and p.wk == g["k_width"]
    assert p.ld == g["fused_width"] == g["q_width"] + g["k_width"] + g["v_width"]
    assert p.ld != 3 * g["q_width"]
    # the oracle normalises Q and K and leaves V byte-identical
    y, yr = oracle.per_head(p.x, p.dtype, p.hq, p.hkv, p.head_dim, p.gamma_q, p.gamma_k, p.eps)
    qk = g["q_width"] + g["k_width"]
    assert np.array_equal(yr[:, qk:], p.x[:, qk:])
    assert (yr[:, :qk] != p.x[:, :qk]).mean() > 0.9


def test_config_shapes():
    p = synth.small_fused_f32()
    assert (p.T, p.ld, p.wq, p.wk, p.dtype) == (4, 3072, 2048, 512, synth.F32)
    p = synth.standalone_heads(T=16, H=48)
    assert (p.T, p.ld, p.wq, p.wk, p.hkv) == (16, 6144, 6144, 0, 0) and p.gamma_k is None
    p = synth.layerwise_rows(T=4)
    assert (p.ld, p.wq, p.wk, p.nshards) == (6144, 4096, 1024, 8)
    p = synth.prefill_rows(T=3)
    assert (p.ld, p.wq, p.wk, p.nshards) == (10240, 8192, 1024, 8)
    ph = synth.prefill_rows(T=3, mode="per_head")
    assert np.array_equal(ph.x, p.x)           # both modes on the same input
    assert (ph.hq, ph.hkv, ph.head_dim) == (64, 8, 128)
    assert p.eps == float(np.float32(1e-6))
