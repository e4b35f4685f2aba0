"""The C-ABI library on the CPU: it loads without a GPU, exports every function
include/fmlp.h declares, and rejects bad arguments with the documented status
before touching any device.  No call here reaches a kernel launch: every call
either fails validation or is an M == 0 no-op, so the suite is safe anywhere."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmlp.h")
LIBPATH = os.path.join(ROOT, "gemm_epilogue_bf16_amd", "libfmlp.so")

OK, E_NULL, E_SHAPE, E_ALIGN, E_ARG, E_WS, E_DEV, E_HIP = range(8)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fmlp_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIBPATH):
        from gemm_epilogue_bf16_amd.build import build

        build()
    import gemm_epilogue_bf16_amd as F

    return F.lib()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("fmlp_linear", "fmlp_mlp2", "fmlp_geglu", "fmlp_moe_geglu"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert L.fmlp_version() >= 100


def test_status_strings(L):
    for s in range(8):
        assert L.fmlp_status_string(s).decode().startswith("FMLP_")


# fake, 16-byte aligned, never dereferenced
X, W, B, Y, WS = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def _err(L):
    return L.fmlp_last_error().decode()


@pytest.mark.parametrize("args,status,msg", [
    ((X, W, None, 0, 4, 30, 8, Y, None), E_ALIGN, "K=30"),
    ((X, W, None, 0, 4, 32, 12, Y, None), E_ALIGN, "N=12"),
    ((X, W, None, 0, 4, 0, 8, Y, None), E_SHAPE, "K=0"),
    ((X, W, None, 0, 4, 1 << 22, 8, Y, None), E_SHAPE, "K=4194304"),
    ((X, W, None, 0, -1, 32, 8, Y, None), E_SHAPE, "M=-1"),
    ((X, W, None, 7, 4, 32, 8, Y, None), E_ARG, "act=7"),
    ((None, W, None, 0, 4, 32, 8, Y, None), E_NULL, "x is NULL"),
    ((X, None, None, 0, 4, 32, 8, Y, None), E_NULL, "W is NULL"),
    ((X, W, None, 0, 4, 32, 8, None, None), E_NULL, "y is NULL"),
    ((X + 2, W, None, 0, 4, 32, 8, Y, None), E_ALIGN, "x is not 16-byte aligned"),
    ((X, W, B + 8, 0, 4, 32, 8, Y, None), E_ALIGN, "b is not 16-byte aligned"),
])
def test_linear_validation(L, args, status, msg):
    assert L.fmlp_linear(*args) == status
    assert msg in _err(L)


def test_linear_zero_rows_is_a_noop(L):
    assert L.fmlp_linear(X, W, None, 0, 0, 32, 8, Y, None) == OK
    # no tokens: activations and outputs may be NULL (empty tensors), weights may not
    assert L.fmlp_linear(None, W, None, 0, 0, 32, 8, None, None) == OK
    assert L.fmlp_linear(None, None, None, 0, 0, 32, 8, None, None) == E_NULL
    assert L.fmlp_linear(X + 2, W, None, 0, 0, 32, 8, Y, None) == E_ALIGN
    assert L.fmlp_mlp2(None, W, B, W, B, 1, 0, 32, 64, 32, None, WS, 1 << 20, None) == OK
    assert L.fmlp_glu(None, W, W, W, 4, 0, 64, 128, None, WS, 1 << 20, None) == OK
    assert L.fmlp_moe_glu(None, None, None, W, W, W, 2, 0, 64, 128, 4, 2, None, WS, 1 << 20, None) == OK
    assert L.fmlp_moe_route(None, W, 0, 64, 4, 2, None, None, None, None) == OK


def test_mlp2_validation(L):
    need = L.fmlp_mlp2_workspace_size(4, 32, 64, 32)
    assert need == 8192 + 512  # 8 KB header + 4*64 bf16 rounded to 256
    # workspace NULL / too small
    assert L.fmlp_mlp2(X, W, B, W, B, 1, 20, 256, 256, 256, Y, None, 0, None) == E_WS
    assert L.fmlp_mlp2(X, W, B, W, B, 1, 20, 256, 256, 256, Y, WS, 100, None) == E_WS
    assert "needs" in _err(L)
    # the small fused path needs no workspace; a forced wrong path is rejected
    assert L.fmlp_set_path(1) == OK
    try:
        assert L.fmlp_mlp2(X, W, B, W, B, 1, 17, 32, 64, 32, Y, WS, 1 << 20, None) == E_ARG
        assert "M <= 16" in _err(L)
    finally:
        L.fmlp_set_path(0)
    assert L.fmlp_set_path(3) == OK
    try:
        assert L.fmlp_mlp2(X, W, B, W, B, 1, 17, 256, 64, 32, Y, WS, 1 << 20, None) == E_ARG
    finally:
        L.fmlp_set_path(0)
    assert L.fmlp_set_path(9) == E_ARG
    assert L.fmlp_mlp2(X, W, B, W, B, 5, 4, 32, 64, 32, Y, WS, 1 << 20, None) == E_ARG
    assert L.fmlp_mlp2(X, W, B, W, B, 1, 4, 32, 60, 32, Y, WS, 1 << 20, None) == E_ALIGN
    assert L.fmlp_mlp2(X, W, B, None, B, 1, 4, 32, 64, 32, Y, WS, 1 << 20, None) == E_NULL


def test_geglu_validation(L):
    need = L.fmlp_geglu_workspace_size(8192, 768, 3072)
    # the larger of m (two launches) and the one-launch form's arrival words +
    # two fp32 partials of y (128 token tiles of 64 rows, 2 parts of the hidden range)
    assert need == 8192 + max(8192 * 3072 * 2, 128 * 8 + 2 * 8192 * 768 * 4)
    assert L.fmlp_geglu_workspace_size(8192, 4096, 3072) == 8192 + 8192 * 3072 * 2   # D > 1024: no fused form
    assert L.fmlp_geglu(X, W, W, W, 16, 64, 128, Y, None, 0, None) == E_WS
    assert L.fmlp_geglu(X, W, W, W, 16, 64, 128, Y, WS + 8, 1 << 20, None) == E_ALIGN
    assert L.fmlp_geglu(X, W, None, W, 16, 64, 128, Y, WS, 1 << 20, None) == E_NULL
    assert L.fmlp_geglu(X, W, W, W, 16, 60, 128, Y, WS, 1 << 20, None) == E_ALIGN
    assert L.fmlp_set_path(3) == OK
    try:
        assert L.fmlp_geglu(X, W, W, W, 16, 64, 128, Y, WS, 1 << 20, None) == E_ARG
    finally:
        L.fmlp_set_path(0)
    assert L.fmlp_geglu(X, W, W, W, 0, 64, 128, Y, WS, 1 << 20, None) == OK
    assert L.fmlp_set_path(4) == OK   # the one-launch gated block: D <= 1024, glu only
    try:
        assert L.fmlp_geglu(X, W, W, W, 16, 1032, 128, Y, WS, 1 << 30, None) == E_ARG
        assert "D <= 1024" in _err(L)
        assert L.fmlp_mlp2(X, W, None, W, None, 2, 16, 64, 128, 64, Y, WS, 1 << 20, None) == E_ARG
    finally:
        L.fmlp_set_path(0)
    assert L.fmlp_set_path(5) == E_ARG
    assert L.fmlp_set_cooperative_decode(2) == E_ARG
    assert L.fmlp_set_cooperative_decode(1) == OK
    assert L.fmlp_set_cooperative_decode(0) == OK


def test_glu_validation(L):
    assert L.fmlp_glu_workspace_size(300, 512, 1024) == L.fmlp_geglu_workspace_size(300, 512, 1024)
    for act in (0, 1, 2, 3, 4):   # every fmlp_act is a valid gate activation; M == 0 is a no-op
        assert L.fmlp_glu(X, W, W, W, act, 0, 64, 128, Y, WS, 1 << 20, None) == OK
    for act in (-1, 5):
        assert L.fmlp_glu(X, W, W, W, act, 16, 64, 128, Y, WS, 1 << 20, None) == E_ARG
        assert "gate_act" in _err(L)
    assert L.fmlp_glu(X, W, W, W, 4, 16, 64, 128, Y, None, 0, None) == E_WS
    ids, gw = 0x60000, 0x70000
    need = L.fmlp_moe_workspace_size(64, 64, 128, 4, 2)
    assert L.fmlp_moe_glu(X, ids, gw, W, W, W, 5, 64, 64, 128, 4, 2, Y, WS, need, None) == E_ARG
    assert L.fmlp_moe_glu(X, ids, gw, W, W, W, 4, 0, 64, 128, 4, 2, Y, WS, need, None) == OK


def test_route_validation(L):
    ids, gw, lg = 0x60000, 0x70000, 0x80000
    assert L.fmlp_moe_route(X, W, 0, 4096, 8, 2, ids, gw, None, None) == OK        # T == 0: no-op
    assert L.fmlp_moe_route(X, W, 16, 4096, 65, 2, ids, gw, None, None) == E_ARG
    assert L.fmlp_moe_route(X, W, 16, 4096, 0, 1, ids, gw, None, None) == E_ARG
    assert L.fmlp_moe_route(X, W, 16, 4096, 8, 9, ids, gw, None, None) == E_ARG
    assert L.fmlp_moe_route(X, W, 16, 4096, 4, 5, ids, gw, None, None) == E_ARG
    assert "top_k" in _err(L)
    assert L.fmlp_moe_route(X, W, 16, 4092, 8, 2, ids, gw, None, None) == E_ALIGN
    assert L.fmlp_moe_route(X, None, 16, 4096, 8, 2, ids, gw, None, None) == E_NULL
    assert L.fmlp_moe_route(X, W, 16, 4096, 8, 2, None, gw, None, None) == E_NULL
    assert L.fmlp_moe_route(X, W, 16, 4096, 8, 2, ids, gw + 2, lg, None) == E_ALIGN


def test_new_acts_accepted(L):
    for act in (3, 4):   # relu, silu
        assert L.fmlp_linear(X, W, None, act, 0, 32, 8, Y, None) == OK
        assert L.fmlp_mlp2(X, W, B, W, B, act, 0, 32, 64, 32, Y, WS, 1 << 20, None) == OK
    assert L.fmlp_linear(X, W, None, 5, 4, 32, 8, Y, None) == E_ARG


def test_moe_validation(L):
    T, D, H, E, k = 4096, 4096, 14336, 8, 2
    P = T * k
    need = L.fmlp_moe_workspace_size(T, D, H, E, k)
    assert need >= 8192 + 3 * P * 4 + P * H * 2 + P * D * 4
    ids, gw = 0x60000, 0x70000
    assert L.fmlp_moe_geglu(X, ids, gw, W, W, W, T, D, H, 0, k, Y, WS, need, None) == E_ARG
    assert L.fmlp_moe_geglu(X, ids, gw, W, W, W, T, D, H, E, 9, Y, WS, need, None) == E_ARG
    assert L.fmlp_moe_geglu(X, None, gw, W, W, W, T, D, H, E, k, Y, WS, need, None) == E_NULL
    assert L.fmlp_moe_geglu(X, ids, gw, W, W, W, T, D, H, E, k, Y, WS, need - 1, None) == E_WS
    assert L.fmlp_moe_geglu(X, ids, gw, W, W, W, T, 4092, H, E, k, Y, WS, need, None) == E_ALIGN
    assert L.fmlp_moe_geglu(X, ids, gw, W, W, W, 0, D, H, E, k, Y, WS, need, None) == OK
    # routed rows are gathered from x with 32-bit byte offsets: x < 2^30 elements
    big_t = (1 << 30) // D
    big_need = L.fmlp_moe_workspace_size(big_t, D, H, E, k)
    assert L.fmlp_moe_geglu(X, ids, gw, W, W, W, big_t, D, H, E, k, Y, WS, big_need, None) == E_SHAPE
    assert "T*D" in _err(L)
    assert L.fmlp_moe_error_offset() < 8192


def test_no_fallback_without_library(tmp_path, monkeypatch):
    """The binding raises when the library is missing: there is no CPU path."""
    import gemm_epilogue_bf16_amd as F

    monkeypatch.setattr(F, "_lib", None)
    monkeypatch.setattr(F, "library_path", lambda: str(tmp_path / "absent.so"))
    with pytest.raises(F.FmlpError, match="not built"):
        F.lib()


def test_w8_validation(L):
    S = 0x90000   # a 4-byte aligned stand-in for a scale array (never dereferenced)
    # h after the untouched 8 KB decode header (a workspace shared with the bf16 calls)
    assert L.fmlp_w8_workspace_size(16, 4096) == 8192 + 16 * 4096 * 2
    assert L.fmlp_w8_workspace_size(1, 4096) == 8192 + 4096 * 4   # one token: H / 2 words of 8 bytes
    assert L.fmlp_w8_workspace_size(0, 4096) == 0
    assert L.fmlp_linear_w8(X, W, S, None, 0, 0, 64, 32, Y, None) == OK          # M == 0: no-op
    assert L.fmlp_linear_w8(X, W, S, None, 0, 17, 64, 32, Y, None) == E_ARG
    assert "M <= 16" in _err(L)
    assert L.fmlp_linear_w8(X, W, S, None, 0, 4, 24, 32, Y, None) == E_ALIGN     # K % 16
    assert "multiple of 16" in _err(L)
    assert L.fmlp_linear_w8(X, W, S, None, 0, 4, 64, 36, Y, None) == E_ALIGN     # N % 8
    assert L.fmlp_linear_w8(X, W, None, None, 0, 4, 64, 32, Y, None) == E_NULL
    assert L.fmlp_linear_w8(X, W, S + 2, None, 0, 4, 64, 32, Y, None) == E_ALIGN
    assert L.fmlp_linear_w8(X, W, S, None, 9, 4, 64, 32, Y, None) == E_ARG
    assert L.fmlp_mlp2_w8(X, W, S, None, W, S, None, 1, 4, 64, 128, 64, Y, None, 0, None) == E_WS
    assert L.fmlp_mlp2_w8(X, W, S, None, W, S, None, 1, 4, 64, 128, 64, Y, WS, 4 * 128 * 2 + 8190, None) == E_WS
    assert L.fmlp_mlp2_w8(X, W, S, None, W, S, None, 1, 0, 64, 128, 64, Y, None, 0, None) == OK
    assert L.fmlp_glu_w8(X, W, S, W, S, W, None, 2, 4, 64, 128, Y, WS, 1 << 20, None) == E_NULL
    assert L.fmlp_glu_w8(X, W, S, W, S, W, S, 2, 17, 64, 128, Y, WS, 1 << 20, None) == E_ARG
    assert L.fmlp_glu_w8(X, W, S, W, S, W, S, 2, 0, 64, 128, Y, WS, 1 << 20, None) == OK


def test_decode_header_words(L):
    """The decode kernel's generation and timeout words sit inside the 8 KB
    header, apart from each other and from the MoE error word."""
    gen, tmo, moe = L.fmlp_decode_generation_offset(), L.fmlp_decode_timeout_offset(), L.fmlp_moe_error_offset()
    assert len({gen, tmo, moe}) == 3
    assert all(o % 4 == 0 and o + 4 <= 8192 for o in (gen, tmo, moe))
    # the FP8 and bf16 two-layer calls share a workspace: both keep data after the header
    assert L.fmlp_mlp2_workspace_size(16, 4096, 4096, 4096) >= 8192 + 16 * 4096 * 2
    assert L.fmlp_w8_workspace_size(16, 4096) >= 8192 + 16 * 4096 * 2


def test_abi_under_host_sanitizers(tmp_path):
    """abi.cpp built for the host alone with AddressSanitizer and
    UndefinedBehaviorSanitizer (kernel launchers stubbed out), driven through
    every entry point with rejected and no-op arguments: every status is the
    documented one and neither sanitizer reports anything."""
    import shutil
    import subprocess

    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs g++ and the ROCm runtime library")
    here = os.path.join(ROOT, "tests", "abi_host")
    exe = str(tmp_path / "abi_san")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "gemm_epilogue_bf16_amd", "csrc", "abi.cpp"),
           os.path.join(here, "stub_launch.cpp"), os.path.join(here, "driver.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ALL OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
