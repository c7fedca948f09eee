"""The C-ABI library on the host: it loads, exports what the header declares,
and rejects bad arguments before any HIP call (CPU only, no kernel runs)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import qk_norm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qknorm.h")

A16 = 0x10000          # a fake, 16-byte aligned "device" address (never dereferenced)
BF16, F32, F16, F8 = q.QKNORM_BF16, q.QKNORM_F32, q.QKNORM_F16, q.QKNORM_FP8_E4M3


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qknorm_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return q.load()


def test_header_declares_the_entry_points():
    assert _declared() == sorted(q.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in _declared():
        assert name in syms, f"{name} not exported with C linkage"


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(QKNORM_[A-Z0-9_]+)\s+(-?\d+)", text))
    for k, v in consts.items():
        if hasattr(q, k):
            assert getattr(q, k) == int(v), k


def test_abi_version_and_strerror(lib):
    assert q.abi_version() == 1
    for code in range(-8, 1):
        s = q.strerror(code)
        assert isinstance(s, str) and s
    assert q.strerror(0) == "success"
    assert "unknown" in q.strerror(12345)


def test_gfx950_code_object_in_library():
    data = open(q.LIB_PATH, "rb").read()
    assert b"gfx950" in data


# ------------------------------------------------------------- validation --

def ph(lib, qkv=A16, T=4, ld=3072, hq=16, hkv=4, D=128, gq=A16, gk=A16, eps=1e-6, dt=F32):
    return lib.qknorm_per_head(qkv, T, ld, hq, hkv, D, gq, gk, eps, dt, None)


def lw(lib, qkv=A16, T=4, ld=6144, wq=4096, wk=1024, gq=A16, gk=A16, eps=1e-6, R=8, dt=BF16):
    return lib.qknorm_layerwise(qkv, T, ld, wq, wk, gq, gk, eps, R, dt, None)


def ps(lib, qkv=A16, T=4, ld=6144, wq=4096, wk=1024, R=8, pq=A16, pk=A16, dt=BF16):
    return lib.qknorm_partial_sumsq(qkv, T, ld, wq, wk, R, pq, pk, dt, None)


def ap(lib, qkv=A16, T=4, ld=6144, wq=4096, wk=1024, pq=A16, pk=A16, n=8, nwq=4096, nwk=1024,
       gq=A16, gk=A16, eps=1e-6, dt=BF16):
    return lib.qknorm_apply_scalar(qkv, T, ld, wq, wk, pq, pk, n, nwq, nwk, gq, gk, eps, dt, None)


@pytest.mark.parametrize("call", [ph, lw, ps, ap], ids=["per_head", "layerwise", "partial", "apply"])
def test_bad_dtype(lib, call):
    assert call(lib, dt=4) == q.QKNORM_E_DTYPE
    assert call(lib, dt=-1) == q.QKNORM_E_DTYPE
    # fp16 and E4M3 are valid codes (T = 0: validated, nothing launched)
    assert call(lib, dt=F16, T=0) == q.QKNORM_OK
    assert call(lib, dt=F8, T=0) == q.QKNORM_OK


@pytest.mark.parametrize("call", [ph, lw, ap], ids=["per_head", "layerwise", "apply"])
@pytest.mark.parametrize("eps", [-1e-6, math.nan, math.inf, -math.inf])
def test_bad_eps(lib, call, eps):
    assert call(lib, eps=eps) == q.QKNORM_E_EPS


def test_zero_eps_is_valid_and_T0_is_a_noop(lib):
    # T == 0: everything valid, nothing launched, no HIP call made
    assert ph(lib, T=0, eps=0.0) == q.QKNORM_OK
    assert lw(lib, T=0) == q.QKNORM_OK
    assert ps(lib, T=0) == q.QKNORM_OK
    assert ap(lib, T=0) == q.QKNORM_OK
    # and with NULL buffers, since nothing would be touched
    assert ph(lib, qkv=None, T=0, gq=None, gk=None) == q.QKNORM_OK
    assert lw(lib, qkv=None, T=0, gq=None, gk=None) == q.QKNORM_OK
    assert ps(lib, qkv=None, T=0, pq=None, pk=None) == q.QKNORM_OK
    assert ap(lib, qkv=None, T=0, pq=None, pk=None, gq=None, gk=None) == q.QKNORM_OK
    # empty widths are no-ops too
    assert ph(lib, hq=0, hkv=0, gq=None, gk=None) == q.QKNORM_OK


def test_shapes(lib):
    assert ph(lib, T=-1) == q.QKNORM_E_SHAPE
    assert ph(lib, hq=-1) == q.QKNORM_E_SHAPE
    assert ph(lib, hkv=-2) == q.QKNORM_E_SHAPE
    assert ph(lib, D=0) == q.QKNORM_E_SHAPE
    assert ph(lib, ld=2559) == q.QKNORM_E_SHAPE            # < (16+4)*128
    assert ph(lib, ld=-4) == q.QKNORM_E_SHAPE
    assert lw(lib, ld=5119) == q.QKNORM_E_SHAPE
    assert lw(lib, wq=-8) == q.QKNORM_E_SHAPE
    assert lw(lib, R=0) == q.QKNORM_E_SHAPE
    assert lw(lib, R=-3) == q.QKNORM_E_SHAPE
    assert lw(lib, R=3) == q.QKNORM_E_SHAPE                # does not divide 4096
    assert lw(lib, wq=4000, R=8) == q.QKNORM_E_ALIGN        # 500 bf16 = 1000 B per shard
    assert ps(lib, R=7) == q.QKNORM_E_SHAPE
    assert ap(lib, n=0) == q.QKNORM_E_SHAPE
    assert ap(lib, nwq=4095) == q.QKNORM_E_SHAPE            # full width below local width
    assert ap(lib, nwk=0) == q.QKNORM_E_SHAPE


def test_null_pointers(lib):
    assert ph(lib, qkv=None) == q.QKNORM_E_NULLPTR
    assert ph(lib, gq=None) == q.QKNORM_E_NULLPTR
    assert ph(lib, gk=None) == q.QKNORM_E_NULLPTR           # hkv > 0 needs gamma_k
    assert lw(lib, qkv=None) == q.QKNORM_E_NULLPTR
    assert lw(lib, gk=None) == q.QKNORM_E_NULLPTR
    assert ps(lib, pq=None) == q.QKNORM_E_NULLPTR
    assert ps(lib, pk=None) == q.QKNORM_E_NULLPTR
    assert ap(lib, pk=None) == q.QKNORM_E_NULLPTR
    assert ap(lib, gq=None) == q.QKNORM_E_NULLPTR


def test_alignment(lib):
    assert ph(lib, qkv=A16 + 8) == q.QKNORM_E_ALIGN
    assert ph(lib, gq=A16 + 4) == q.QKNORM_E_ALIGN
    assert ph(lib, ld=3073) == q.QKNORM_E_ALIGN             # pitch 12292 B
    assert lw(lib, ld=6145) == q.QKNORM_E_ALIGN
    assert lw(lib, gq=A16 + 2) == q.QKNORM_E_ALIGN
    assert ps(lib, pq=A16 + 1) == q.QKNORM_E_ALIGN
    assert ap(lib, pk=A16 + 2) == q.QKNORM_E_ALIGN
    assert ap(lib, wq=4092, nwq=4096) == q.QKNORM_E_ALIGN  # Q/K boundary off a 16 B vector
    # E4M3: one byte per element, so 16-byte rules count 16 elements
    assert lw(lib, ld=6152, dt=F8) == q.QKNORM_E_ALIGN     # pitch 6152 B
    assert lw(lib, wq=4096 + 8, ld=6160, R=1, dt=F8) == q.QKNORM_E_ALIGN
    assert lw(lib, wq=4096, wk=1024, R=128, dt=F8) == q.QKNORM_E_ALIGN   # 8-byte K shards
    assert lw(lib, T=0, ld=6160, dt=F8) == q.QKNORM_OK


@pytest.mark.parametrize("dt,D", [(F32, 4), (F32, 12), (F32, 16), (F32, 100), (F32, 256),
                                  (BF16, 8), (BF16, 24), (BF16, 96), (BF16, 128), (BF16, 504),
                                  (BF16, 512), (F16, 40), (F16, 128), (F16, 512),
                                  (F8, 16), (F8, 48), (F8, 128), (F8, 1008), (F8, 1024)])
def test_head_widths_accepted(lib, dt, D):
    # any head of 16 to 1024 bytes in 16-byte steps (T = 0: validated, nothing launched)
    assert ph(lib, T=0, D=D, ld=20 * D, dt=dt) == q.QKNORM_OK


def test_head_bytes_not_a_multiple_of_16(lib):
    assert ph(lib, T=0, D=100, ld=20 * 100, dt=BF16) == q.QKNORM_E_ALIGN   # 200-byte heads
    assert ph(lib, D=100, ld=20 * 100, dt=BF16) == q.QKNORM_E_ALIGN
    assert ph(lib, D=2, hq=8, hkv=0, ld=16, dt=F32) == q.QKNORM_E_ALIGN    # 8-byte heads
    assert ph(lib, D=20, hq=4, hkv=0, ld=80, dt=F8) == q.QKNORM_E_ALIGN


def test_unsupported(lib):
    assert ph(lib, D=512, ld=20 * 512) == q.QKNORM_E_UNSUPPORTED      # fp32: 2 KiB heads
    assert ph(lib, D=512, ld=20 * 512, T=0) == q.QKNORM_E_UNSUPPORTED  # checked before T == 0
    assert ph(lib, D=1024, ld=20 * 1024, dt=F16) == q.QKNORM_E_UNSUPPORTED
    assert ph(lib, D=2048, ld=20 * 2048, dt=F8) == q.QKNORM_E_UNSUPPORTED
    # one 16-byte head per 32 MiB row: a trip of 128 heads would span 4 GiB
    assert ph(lib, D=8, hq=1, hkv=0, ld=1 << 24, dt=BF16, T=0) == q.QKNORM_E_UNSUPPORTED
    assert ph(lib, D=8, hq=1, hkv=0, ld=1 << 20, dt=BF16, T=0) == q.QKNORM_OK
    assert lw(lib, R=2048, wq=4096 * 8, wk=2048 * 8, ld=6144 * 8) == q.QKNORM_E_UNSUPPORTED
    assert ap(lib, n=4096) == q.QKNORM_E_UNSUPPORTED
    # rows are addressed with 32-bit offsets: pitch above 64 MiB is refused
    assert ph(lib, ld=(1 << 24) + 4, T=2) == q.QKNORM_E_UNSUPPORTED      # fp32: 64 MiB + 16 B
    assert lw(lib, ld=(1 << 25) + 8, T=2) == q.QKNORM_E_UNSUPPORTED      # bf16


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    g = torch.ones(128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        q.qknorm_per_head(x, 2, 0, 128, g)
    with pytest.raises(ValueError, match="GPU"):
        q.qknorm_layerwise(x, 256, 0, torch.ones(256, dtype=torch.bfloat16))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        q.load(str(tmp_path / "nope.so"))


def pj(lib, x=A16, ldx=256, w=A16, ldw=256, out=A16, ld=768, T=4, hidden=256, hq=2, hkv=2,
       D=128, gq=A16, gk=A16, eps=1e-6, flags=0, dt=BF16):
    return lib.qknorm_qkv_proj_per_head(x, ldx, w, ldw, out, ld, T, hidden, hq, hkv, D, gq, gk,
                                        eps, flags, dt, None)


def test_projection_validation(lib):
    # everything valid with T = 0: validated, nothing launched
    assert pj(lib, T=0) == q.QKNORM_OK
    assert pj(lib, T=0, D=64, ld=384) == q.QKNORM_OK
    assert pj(lib, T=0, flags=q.QKNORM_PROJ_PLAIN, gq=None, gk=None) == q.QKNORM_OK
    assert pj(lib, T=0, dt=F16) == q.QKNORM_OK                 # bf16 and fp16
    assert pj(lib, dt=F32) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, dt=F8) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, dt=7) == q.QKNORM_E_DTYPE
    assert pj(lib, flags=2) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, hidden=96, ldx=96, ldw=96) == q.QKNORM_E_UNSUPPORTED     # K step of 64
    assert pj(lib, T=0, D=256, ld=1536) == q.QKNORM_OK                     # head_dim 64, 128, 256
    assert pj(lib, D=96, ld=576) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, D=512, ld=3072) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, ld=767) == q.QKNORM_E_SHAPE                             # ld < N = 768
    assert pj(lib, ldx=128) == q.QKNORM_E_SHAPE                            # ldx < hidden
    assert pj(lib, hidden=0) == q.QKNORM_E_SHAPE
    assert pj(lib, hq=-1) == q.QKNORM_E_SHAPE
    assert pj(lib, x=None) == q.QKNORM_E_NULLPTR
    assert pj(lib, out=None) == q.QKNORM_E_NULLPTR
    assert pj(lib, gk=None) == q.QKNORM_E_NULLPTR
    assert pj(lib, w=A16 + 2) == q.QKNORM_E_ALIGN
    assert pj(lib, ld=772) == q.QKNORM_E_ALIGN                             # 1544-byte pitch
    assert pj(lib, eps=-1.0) == q.QKNORM_E_EPS
    assert pj(lib, ldx=(1 << 22) + 8, T=0) == q.QKNORM_E_UNSUPPORTED       # 256 rows over 2 GiB
    assert pj(lib, ldw=(1 << 22) + 8, T=0) == q.QKNORM_E_UNSUPPORTED


def pjw(lib, ws=A16, wsb=1 << 30, x=A16, ldx=256, w=A16, ldw=256, out=A16, ld=768, T=4, hidden=256,
        hq=2, hkv=2, D=128, gq=A16, gk=A16, eps=1e-6, flags=0, dt=BF16):
    return lib.qknorm_qkv_proj_per_head_ws(x, ldx, w, ldw, out, ld, T, hidden, hq, hkv, D, gq, gk,
                                           eps, flags, dt, ws, wsb, None)


def test_projection_workspace_size_and_validation(lib):
    f = lib.qknorm_qkv_proj_workspace_bytes
    N = (32 + 2 * 8) * 128                                 # a Qwen3-8B layer
    assert f(1, 32, 8, 128) == 4 * 1 * N * 4               # up to 8 tokens: 4 slices of K
    assert f(8, 32, 8, 128) == 4 * 8 * N * 4
    assert f(9, 32, 8, 128) == 8 * 9 * N * 4               # 9 to 16: 8 slices
    assert f(16, 32, 8, 128) == 8 * 16 * N * 4
    assert f(17, 32, 8, 128) == 8 * 17 * N * 4             # 17 to 32: 8 slices
    assert f(64, 32, 8, 128) == 4 * 64 * N * 4             # 33 to 64: 4 slices
    assert f(1, 1, 1, 1) == 256                            # 48 bytes, rounded up to 256
    assert f(0, 32, 8, 128) == 0 and f(65, 32, 8, 128) == 0 and f(4096, 32, 8, 128) == 0
    assert f(-1, 1, 0, 64) == q.QKNORM_E_SHAPE
    assert f(1, -1, 0, 64) == q.QKNORM_E_SHAPE
    assert f(1, 1, 0, 0) == q.QKNORM_E_SHAPE
    m = (1 << 31) - 1
    assert f(1, m, m, m) == q.QKNORM_E_UNSUPPORTED
    assert f(1 << 40, 1, 0, 64) == q.QKNORM_E_UNSUPPORTED
    # the workspace form: the projection's own checks first, then the workspace's
    need = 4 * 4 * 768 * 4
    assert pjw(lib, dt=F32) == q.QKNORM_E_UNSUPPORTED
    assert pjw(lib, ld=767) == q.QKNORM_E_SHAPE
    assert pjw(lib, x=None) == q.QKNORM_E_NULLPTR
    assert pjw(lib, ws=None, wsb=need) == q.QKNORM_E_NULLPTR
    assert pjw(lib, ws=A16 + 8, wsb=need) == q.QKNORM_E_ALIGN
    assert pjw(lib, wsb=need - 1) == q.QKNORM_E_SHAPE
    assert pjw(lib, wsb=-1) == q.QKNORM_E_SHAPE
    assert pjw(lib, T=0, ws=None, wsb=0) == q.QKNORM_OK   # validated, nothing launched
    assert pjw(lib, T=0, ws=None, wsb=-1) == q.QKNORM_E_SHAPE


def test_sizes_whose_products_overflow_64_bits_are_rejected(lib):
    # pitches, widths and head counts near the int64 / int32 limits: each is
    # rejected by value, before any product of it is formed (a product that
    # wrapped could pass a bound and reach a kernel with truncated offsets)
    big = 1 << 62
    assert lw(lib, ld=big, wq=big, wk=big) == q.QKNORM_E_SHAPE            # wq + wk > ld
    assert ps(lib, ld=big, wq=big - 1024, wk=2048, R=1) == q.QKNORM_E_SHAPE
    assert lw(lib, ld=big, wq=4096, wk=1024) == q.QKNORM_E_UNSUPPORTED     # pitch past 64 MiB
    assert ph(lib, ld=big, dt=F32) == q.QKNORM_E_UNSUPPORTED                # ld * 4 would wrap to 0
    assert ph(lib, ld=(1 << 63) - 16, dt=BF16) == q.QKNORM_E_UNSUPPORTED
    assert ap(lib, ld=big, wq=4096, wk=1024) == q.QKNORM_E_UNSUPPORTED
    # projection: 256 rows of a 2^61-element pitch wrap a 64-bit byte count to 0
    assert pj(lib, ldx=1 << 61) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, ldw=1 << 61) == q.QKNORM_E_UNSUPPORTED
    assert pj(lib, ld=1 << 61) == q.QKNORM_E_UNSUPPORTED
    # (hq + 2 hkv) * head_dim past int64 from int32 arguments
    m = (1 << 31) - 1
    assert pj(lib, hq=m, hkv=m, D=m, ld=big) == q.QKNORM_E_SHAPE           # N > ld
    assert pj(lib, hq=m, hkv=m, D=128, ld=big) == q.QKNORM_E_UNSUPPORTED


def _c_program():
    """tests/c_abi/closed_form, built with gcc here if it is not there yet."""
    import importlib.util
    path = os.path.join(ROOT, "tests", "c_abi", "build.py")
    spec = importlib.util.spec_from_file_location("c_abi_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.BIN if os.path.exists(mod.BIN) else mod.build()


def test_plain_c_program_gets_the_validation_codes():
    # a C program linked against the library (no Python in between) gets every
    # validation code before any HIP call; its GPU part runs in the GPU tests
    res = subprocess.run([_c_program(), "--validation-only"], capture_output=True, text=True,
                         timeout=60)
    assert res.returncode == 0, res.stderr
    assert "validation codes ok" in res.stdout


def test_python_call_module_forwards_to_the_same_library(lib):
    # the binding's call path (qk_norm_amd/csrc/pyfast.cpp) converts the Python
    # arguments itself and calls the same extern "C" functions: the library's
    # validation codes come back unchanged, and the process holds one copy of
    # the library whichever way it was opened
    from qk_norm_amd import _qknorm_fast as f
    assert f.per_head(A16, 4, 6144, 48, 0, 128, A16, None, 1e-6, 99, None) == q.QKNORM_E_DTYPE
    assert f.per_head(0, 4, 6144, 48, 0, 128, A16, None, 1e-6, BF16, None) == q.QKNORM_E_NULLPTR
    assert f.layerwise(A16, 4, 6144, 4096, 1024, A16, A16, 1e-6, 3, BF16, None) == q.QKNORM_E_SHAPE
    assert f.partial_sumsq(A16, 4, 6144, 4096, 1024, 0, A16, A16, BF16, None) == q.QKNORM_E_SHAPE
    assert f.apply_scalar(A16, 4, 6144, 4096, 1024, None, None, 8, 4096, 1024, A16, A16, 1e-6, BF16,
                          None) == q.QKNORM_E_NULLPTR
    assert f.qkv_proj_per_head(A16, 4096, A16, 4096, A16, 6144, 16, 4096, 32, 8, 128, A16, A16, 1e-6, 0,
                               F32, None) == q.QKNORM_E_UNSUPPORTED
    assert f.per_head(A16, 0, 6144, 48, 0, 128, A16, None, float("nan"), BF16, None) == q.QKNORM_E_EPS
    assert f.qkv_proj_per_head_ws(A16, 4096, A16, 4096, A16, 6144, 16, 4096, 32, 8, 128, A16, A16, 1e-6,
                                  0, BF16, None, 1 << 30, None) == q.QKNORM_E_NULLPTR
    with pytest.raises(TypeError):
        f.per_head(A16, 4)
    with pytest.raises(OverflowError):
        f.per_head(A16, 4, 6144, 1 << 40, 0, 128, A16, None, 1e-6, BF16, None)
    assert q._calls() is f
    maps = {line.split()[-1] for line in open("/proc/self/maps") if "libqknorm.so" in line}
    assert maps == {os.path.realpath(q.LIB_PATH)}, maps


def test_tensor_calls_leave_other_inputs_to_the_python_path(lib):
    # per_head_t / layerwise_t take the common case only (a plain
    # torch.Tensor on the GPU); for anything else they return None without
    # touching the library, and the binding's Python path raises its own error
    import numpy as np
    import torch
    c = q._calls()
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    g = torch.ones(128, dtype=torch.bfloat16)

    class Sub(torch.Tensor):
        pass

    for obj in (x, np.zeros((4, 256), np.float32), x.as_subclass(Sub), [[0.0] * 256] * 4, None):
        assert c.per_head_t(obj, 2, 0, 128, g, None, 1e-6, None) is None
        assert c.layerwise_t(obj, 128, 128, g, g, 1e-6, 1, None) is None
    with pytest.raises(ValueError, match="GPU tensor"):
        q.qknorm_per_head(x, 2, 0, 128, g)
    with pytest.raises(TypeError):
        c.per_head_t(x, 2, 0)
