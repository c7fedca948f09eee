"""Build the gfx950 HIP libraries in-tree: qk_norm_amd/libqknorm.so (the
QK-Norm C ABI) and qk_norm_amd/libqknorm_ceiling.so (the bench's bandwidth
ceiling probes, loaded by bench.py only); and the CPython module
qk_norm_amd/_qknorm_fast*.so that the binding calls the C ABI through.

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
FAST_SOURCE = os.path.join(CSRC, "pyfast.cpp")
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
    # the library's own file name as its SONAME: one copy in a process whether it
    # is opened by path (ctypes) or found by name (the Python call module)
    cmd = [HIPCC, *FLAGS, f"-Wl,-soname,{os.path.basename(out)}", *[f"-D{d}" for d in defs], "-o", tmp,
           *(sources or SOURCES)]
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


def fast_module_path() -> str:
    import sysconfig
    return os.path.join(HERE, "_qknorm_fast" + sysconfig.get_config_var("EXT_SUFFIX"))


def build_fast(verbose: bool = False) -> str:
    """The CPython module that calls the C ABI directly (host C++, g++), linked
    against libqknorm.so in the same directory and against torch's libraries
    (it reads torch tensors through torch's C++ API)."""
    import sysconfig
    import torch
    import torch.utils.cpp_extension as ce
    out = fast_module_path()
    tmp = out + ".tmp"
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    inc = [f for p in ce.include_paths() for f in ("-I", p)]
    libdir = ce.library_paths()[0]
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
           "-I", sysconfig.get_paths()["include"], "-I", os.path.join(ROOT, "include"), *inc,
           "-o", tmp, FAST_SOURCE, "-L", HERE, "-l:libqknorm.so", "-L", libdir, "-ltorch_python", "-ltorch",
           "-lc10", f"-Wl,-rpath,$ORIGIN:{libdir}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("g++ failed building the QK-Norm Python call module")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling(verbose=True))
    print(build_fast(verbose=True))
