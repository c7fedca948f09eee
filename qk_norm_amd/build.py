"""Build the gfx950 HIP libraries in-tree: qk_norm_amd/libqknorm.so (the
QK-Norm C ABI) and qk_norm_amd/libqknorm_ceiling.so (the bench's bandwidth
ceiling probes, loaded by bench.py only).

    python -m qk_norm_amd.build            # or __graft_entry__.build()

Extra -D definitions (launch tuning) can be passed with QKNORM_DEFINES, e.g.
QKNORM_DEFINES="QKNORM_NT=0 QKNORM_PH_UNROLL=2", and another output path
with the ``out`` argument (used for side-by-side variants).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "qknorm_api.hip"), os.path.join(CSRC, "qknorm_kernels.hip"),
           os.path.join(CSRC, "qknorm_proj.hip")]
LIB = os.path.join(HERE, "libqknorm.so")
CEILING_SOURCES = [os.path.join(CSRC, "ceiling_probe.hip")]
CEILING_LIB = os.path.join(HERE, "libqknorm_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                      # every fma in the kernels is written out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = LIB, defines: list[str] | None = None, verbose: bool = False,
          sources: list[str] | None = None) -> str:
    defs = list(defines or [])
    defs += os.environ.get("QKNORM_DEFINES", "").split()
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defs], "-o", tmp, *(sources or SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the QK-Norm library")
    os.replace(tmp, out)
    return out


def build_ceiling(verbose: bool = False) -> str:
    return build(CEILING_LIB, verbose=verbose, sources=CEILING_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling(verbose=True))
