"""Plausible mistakes in the fused projection oracle must fail a pin.

Each mutant is a copy of oracle.qkv_proj_per_head with one change, swapped in
for the real function while the projection pins run (CPU only).
"""
import numpy as np
import pytest

import oracle
import pins


def _make(change):
    def proj(x, w, dtype, hq, hkv, head_dim, gamma_q, gamma_k, eps, norm=True):
        xd, wd = oracle.decode(x, dtype), oracle.decode(w, dtype)
        T, D = xd.shape[0], head_dim
        acc = xd @ wd.T if change != "weight_not_transposed" else (xd @ wd.reshape(wd.shape[1], -1))
        y = acc.copy()
        if norm:
            gd = oracle.gamma_dtype(dtype)
            regions = [(0, hq, gamma_q), (hq * D, hkv, gamma_k)]
            if change == "k_uses_gamma_q":
                regions[1] = (hq * D, hkv, gamma_q)
            if change == "k_offset_zero":
                regions[1] = (0, hkv, gamma_k)
            if change == "v_normalised":
                regions.append(((hq + hkv) * D, hkv, gamma_k))
            for c0, nh, g in regions:
                if nh == 0:
                    continue
                seg = acc[:, c0:c0 + nh * D].reshape(T, nh, D)
                div = nh * D if change == "mean_over_region" else D
                ms = np.sum(seg * seg, axis=-1, keepdims=True) / div
                root = np.sqrt(ms) + eps if change == "eps_outside_root" else np.sqrt(ms + eps)
                gv = oracle.decode(g, gd)
                if change == "gamma_reversed":
                    gv = gv[::-1]
                y[:, c0:c0 + nh * D] = (seg * gv / root).reshape(T, nh * D)
        return y, oracle.round_to(y, dtype)
    return proj


MUTANTS = ["weight_not_transposed", "k_uses_gamma_q", "k_offset_zero", "v_normalised",
           "mean_over_region", "eps_outside_root", "gamma_reversed"]


@pytest.mark.parametrize("change", MUTANTS)
def test_projection_mutant_is_caught(change, monkeypatch):
    monkeypatch.setattr(oracle, "qkv_proj_per_head", _make(change))
    failed = []
    for check in pins.PROJ_CHECKS:
        try:
            check()
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {change} passed every projection pin"


def test_unmutated_copy_passes(monkeypatch):
    # the copy the mutants start from is the real definition
    monkeypatch.setattr(oracle, "qkv_proj_per_head", _make(None))
    for check in pins.PROJ_CHECKS:
        check()
