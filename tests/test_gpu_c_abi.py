"""The library from a plain C program on the GPU: hipMalloc'd buffers, the C
entry points, closed-form results (tests/c_abi/closed_form.c says which)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "closed_form")


def test_plain_c_program_closed_forms():
    # built by __graft_entry__.build(), never inside a GPU run
    assert os.path.exists(BIN), f"{BIN} is not built (run __graft_entry__.build())"
    print(f"[c-abi] {BIN}", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    assert res.returncode == 0, f"exit {res.returncode}: {res.stderr.strip()}"
    for line in ("validation codes ok", "per-head closed forms ok", "layerwise closed forms ok",
                 "projection closed forms ok"):
        assert line in res.stdout, res.stdout
