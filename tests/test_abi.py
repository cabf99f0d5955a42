"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/awq.h, and rejects invalid arguments with the documented
status before launching anything (so fake pointers are never dereferenced).
"""
import ctypes
import os
import re

import pytest

from weight_only_quantization_pack_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5

P = ctypes.c_void_p(0x10000)       # aligned fake device pointers (never used)
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
P4 = ctypes.c_void_p(0x40000)
P5 = ctypes.c_void_p(0x50000)
MIS = ctypes.c_void_p(0x10008)     # 8-byte aligned only
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for must in ["awq_quantize_pack", "awq_search_scale", "awq_search_workspace_bytes",
                 "awq_search_workspace_bytes_fused",
                 "awq_gemv", "awq_gemm", "awq_scale_activations", "awq_status_str"]:
        assert must in names


def test_header_compiles_as_c_and_beside_hip():
    """The header is plain C (C11) and agrees with HIP's own hipStream_t when
    both are included (a conflicting typedef would not compile)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no host C compiler")
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    hip_inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(hip_inc, "hip", "hip_runtime_api.h")):
        pytest.skip("no HIP headers")
    src = '#include <hip/hip_runtime_api.h>\n#include "awq.h"\nint main(void) { hipStream_t s = 0; return (int)awq_status_str(AWQ_OK)[0] + (s != 0); }\n'
    r = subprocess.run([shutil.which("g++") or "g++", "-std=c++17", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        f"-I{hip_inc}", f"-I{os.path.dirname(HEADER)}", "-x", "c++", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sorted(n for n, _, _ in B.SIGNATURES) == header_functions()


def test_status_strings(lib):
    for code, name in B.STATUS.items():
        assert lib.awq_status_str(code).decode() == name
    assert lib.awq_status_str(99).decode() == "AWQ_ERR_UNKNOWN"


def test_format_helpers(lib):
    assert lib.awq_pack_format_version() == 3
    assert lib.awq_packed_words(4096, 4096, 4) == 4096 * 512
    assert lib.awq_packed_words(37, 384, 4) == 48 * 48
    assert lib.awq_packed_words(37, 384, 3) == 48 * 36
    assert lib.awq_packed_words(1, 128, 3) == 16 * 12
    assert lib.awq_packed_words_per_row(4096, 4) == 512
    assert lib.awq_packed_words_per_row(4096, 3) == 384
    assert lib.awq_packed_words_per_row(4096, 2) == 0
    assert lib.awq_packed_words_per_row(0, 4) == 0


def test_search_workspace_size(lib):
    T, N, K, A = 512, 4096, 4096, 20
    need = lib.awq_search_workspace_bytes(T, N, K, A)
    # D of one chunk of alphas (4 x 33.5 MB fit the 128 MB chunk budget) + scales
    assert need >= 4 * N * K * 2 + (2 * A + 1) * K * 4
    assert need < 5 * N * K * 2
    # a D larger than the budget runs one alpha at a time
    big = lib.awq_search_workspace_bytes(T, 28672, 8192, A)
    assert 28672 * 8192 * 2 <= big < 2 * 28672 * 8192 * 2
    # fused path: s_x, s_alpha and 1/s_alpha, and one fp64 loss partial per
    # alpha and 256 x 128 output block; W - w_hat / s stays in registers
    fused = lib.awq_search_workspace_bytes_fused(T, N, K, A)
    partials = A * ((N + 127) // 128) * ((T + 255) // 256) * 8
    assert (2 * A + 1) * K * 4 + partials <= fused < A * N * K * 2 // 100
    assert lib.awq_search_workspace_bytes_fused(0, N, K, A) == 0
    assert lib.awq_search_workspace_bytes(0, N, K, A) == 0
    assert lib.awq_search_workspace_bytes(T, N, K, 0) == 0


def qp(lib, W=P, s=NUL, N=256, K=512, bits=4, gs=128, zp=1, qw=P2, sc=P3, ze=P4):
    return lib.awq_quantize_pack(W, s, N, K, bits, gs, zp, qw, sc, ze, NUL)


def test_quantize_pack_validation(lib):
    assert qp(lib, bits=2) == UNSUP
    assert qp(lib, bits=8) == UNSUP
    assert qp(lib, gs=32) == UNSUP
    assert qp(lib, gs=64, W=NUL) == NULL            # 64-wide groups are supported
    assert qp(lib, zp=2) == UNSUP
    assert qp(lib, zp=0, W=NUL) == NULL            # zero_point 0 (symmetric) is supported
    assert qp(lib, K=500) == SHAPE
    assert qp(lib, K=0) == SHAPE
    assert qp(lib, N=-1) == SHAPE
    assert qp(lib, W=NUL) == NULL
    assert qp(lib, qw=NUL) == NULL
    assert qp(lib, W=MIS) == ALIGN
    assert qp(lib, s=MIS) == ALIGN
    assert qp(lib, W=NUL, qw=MIS) == NULL          # NULL reported before alignment
    assert qp(lib, N=0, W=NUL) == OK               # empty call: nothing to do


def mm(lib, fn, x=P, qw=P2, sc=P3, ze=P4, y=P5, M=1, N=256, K=512, bits=4, gs=128):
    return getattr(lib, fn)(x, qw, sc, ze, y, M, N, K, bits, gs, NUL)


@pytest.mark.parametrize("fn", ["awq_gemv", "awq_gemm"])
def test_matmul_validation(lib, fn):
    assert mm(lib, fn, bits=5) == UNSUP
    assert mm(lib, fn, gs=32) == UNSUP
    assert mm(lib, fn, gs=64, x=NUL) == NULL
    assert mm(lib, fn, K=129) == SHAPE
    assert mm(lib, fn, N=-4) == SHAPE
    assert mm(lib, fn, M=-1) == SHAPE
    assert mm(lib, fn, y=NUL) == NULL
    assert mm(lib, fn, sc=MIS) == ALIGN
    assert mm(lib, fn, M=0, x=NUL) == OK
    assert mm(lib, fn, N=0, x=NUL) == OK


def test_gemv_and_gemm_specific_limits(lib):
    assert mm(lib, "awq_gemv", M=17) == UNSUP
    assert mm(lib, "awq_gemm", bits=3, x=NUL) == NULL             # int3 prefill is supported
    assert mm(lib, "awq_gemv", M=17, bits=3, x=NUL) == UNSUP
    assert mm(lib, "awq_gemm", M=1 << 20, K=4096) == SHAPE      # 32-bit offset limit
    # decode: packed weight >= 2^31 bytes (int4: N*K >= 2^32) or x >= 2^31 bytes
    assert mm(lib, "awq_gemv", M=1, N=1 << 16, K=1 << 16) == SHAPE
    assert mm(lib, "awq_gemv", M=1, N=1 << 16, K=(1 << 16) - 128, x=NUL) == NULL   # just below: passes
    assert mm(lib, "awq_gemv", M=16, N=16, K=1 << 26) == SHAPE


def _scaled(lib, x=P, inv_s=P5, qw=P2, sc=P3, ze=P4, y=P, M=1, N=64, K=256, bits=4, gs=128):
    return lib.awq_gemv_scaled(x, inv_s, qw, sc, ze, y, M, N, K, bits, gs, NUL)


def _gate_up(lib, x=P, inv_s=P5, g=(P2, P3, P4), u=(P2, P3, P4), h=P, M=1, N=64, K=256, bits=4,
             gs=128):
    return lib.awq_gemv_gate_up(x, inv_s, *g, *u, h, M, N, K, bits, gs, NUL)


def test_gemv_scaled_validation(lib):
    assert _scaled(lib, inv_s=NUL) == NULL            # the scaled entry point needs its scale
    assert _scaled(lib, inv_s=MIS) == ALIGN
    assert _scaled(lib, bits=5) == UNSUP
    assert _scaled(lib, gs=32) == UNSUP
    assert _scaled(lib, M=17) == UNSUP
    assert _scaled(lib, K=129) == SHAPE
    assert _scaled(lib, M=-1) == SHAPE
    assert _scaled(lib, M=1, N=1 << 16, K=1 << 16) == SHAPE
    assert _scaled(lib, y=NUL) == NULL
    assert _scaled(lib, M=0, x=NUL) == OK
    assert _scaled(lib, N=0, inv_s=NUL) == OK


def test_gemv_gate_up_validation(lib):
    assert _gate_up(lib, u=(NUL, P3, P4)) == NULL
    assert _gate_up(lib, g=(P2, NUL, P4)) == NULL
    assert _gate_up(lib, h=NUL) == NULL
    assert _gate_up(lib, u=(P2, P3, MIS)) == ALIGN
    assert _gate_up(lib, inv_s=MIS) == ALIGN
    assert _gate_up(lib, inv_s=NUL, x=NUL) == NULL    # inv_s is optional, x is not
    assert _gate_up(lib, bits=2) == UNSUP
    assert _gate_up(lib, gs=256) == UNSUP
    assert _gate_up(lib, M=17) == UNSUP
    assert _gate_up(lib, K=200) == SHAPE
    assert _gate_up(lib, N=-1) == SHAPE
    assert _gate_up(lib, M=16, N=16, K=1 << 26) == SHAPE
    assert _gate_up(lib, M=0, x=NUL, h=NUL) == OK


def test_dequantize_validation(lib):
    f = lib.awq_dequantize
    assert f(P, P2, P3, P4, 64, 256, 5, 128, NUL) == UNSUP
    assert f(P, P2, P3, P4, 64, 256, 4, 32, NUL) == UNSUP
    assert f(P, P2, P3, P4, 64, 200, 4, 128, NUL) == SHAPE
    assert f(P, P2, P3, P4, -1, 256, 4, 128, NUL) == SHAPE
    assert f(NUL, P2, P3, P4, 64, 256, 4, 128, NUL) == NULL
    assert f(P, P2, P3, NUL, 64, 256, 3, 64, NUL) == NULL
    assert f(P, P2, MIS, P4, 64, 256, 4, 128, NUL) == ALIGN
    assert f(NUL, NUL, NUL, NUL, 0, 256, 4, 128, NUL) == OK


def test_gemm_splitk_validation(lib):
    # without a GPU the library assumes 256 compute units: the 64 tiles (64 rows
    # x 128 columns) of a 64 x 8192 output leave most idle, so K = 28672 (224
    # groups) is split 256 / 64 = 4 ways
    need = lib.awq_gemm_splitk_workspace_bytes(64, 8192, 28672)
    assert need == 4 * 64 * 8192 * 4
    assert lib.awq_gemm_splitk_workspace_bytes(2048, 14336, 4096) == 0      # enough tiles
    assert lib.awq_gemm_splitk_workspace_bytes(64, 8192, 1000) == 0         # invalid K
    f = lib.awq_gemm_splitk
    assert f(P, P2, P3, P4, P5, 64, 8192, 28672, 4, 128, P, need - 1, NUL) == WS
    assert f(P, P2, P3, P4, P5, 64, 8192, 28672, 4, 128, NUL, need, NUL) == NULL
    assert f(P, P2, P3, P4, P5, 64, 8192, 28672, 4, 128, MIS, need, NUL) == ALIGN
    assert f(P, P2, P3, P4, P5, 64, 8192, 28672, 2, 128, P, need, NUL) == UNSUP
    assert f(P, P2, P3, P4, P5, 64, 8192, 1000, 4, 128, P, need, NUL) == SHAPE
    assert f(NUL, NUL, NUL, NUL, NUL, 0, 8192, 28672, 4, 128, NUL, 0, NUL) == OK   # empty


def test_search_mlp_validation(lib):
    f = lib.awq_search_scale_mlp
    a = (ctypes.c_float * 2)(0.0, 0.5)
    A = ctypes.cast(a, ctypes.c_void_p)
    W = ctypes.c_void_p(0x60000)
    need = lib.awq_search_mlp_workspace_bytes(64, 256, 384, 200, 2)
    assert need > 0
    assert lib.awq_search_mlp_workspace_bytes(64, 256, 300, 200, 2) == 0     # I % 128 != 0
    args = lambda **kw: [kw.get("wg", P), kw.get("wu", P2), kw.get("wd", P3), kw.get("x", P4),
                         kw.get("T", 64), kw.get("K", 256), kw.get("I", 384), kw.get("K_out", 200),
                         kw.get("al", A), kw.get("na", 2), kw.get("bits", 4), 128, 1, P5, NUL, NUL,
                         kw.get("ws", W), kw.get("wsb", need), NUL]
    assert f(*args(bits=5)) == UNSUP
    assert f(*args(na=0)) == UNSUP
    assert f(*args(T=9000)) == UNSUP
    assert f(*args(I=300)) == SHAPE
    assert f(*args(K=200)) == SHAPE
    assert f(*args(K_out=0)) == SHAPE
    assert f(*args(al=NUL)) == NULL
    assert f(*args(wd=NUL)) == NULL
    assert f(*args(x=MIS)) == ALIGN
    assert f(*args(wsb=need - 1)) == WS


def test_gemm_scaled_validation(lib):
    f = lib.awq_gemm_scaled
    W = ctypes.c_void_p(0x60000)
    assert f(P, NUL, P2, P3, P4, P5, 64, 512, 512, 4, 128, NUL, 0, NUL) == NULL     # inv_s required
    assert f(P, MIS, P2, P3, P4, P5, 64, 512, 512, 4, 128, NUL, 0, NUL) == ALIGN
    assert f(P, P, P2, P3, P4, P5, 64, 512, 500, 4, 128, NUL, 0, NUL) == SHAPE
    assert f(P, P, P2, P3, P4, P5, 64, 512, 512, 5, 128, NUL, 0, NUL) == UNSUP
    # a workspace that is given must hold the split's partials
    need = lib.awq_gemm_splitk_workspace_bytes(64, 512, 8192)
    assert need > 0
    assert f(P, P, P2, P3, P4, P5, 64, 512, 8192, 4, 128, W, need - 16, NUL) == WS
    assert f(P, P, P2, P3, P4, P5, 64, 512, 8192, 4, 128, MIS, need, NUL) == ALIGN
    assert f(NUL, NUL, NUL, NUL, NUL, NUL, 0, 512, 512, 4, 128, NUL, 0, NUL) == OK


def test_gemm_splitk_noalloc_validation(lib):
    f = lib.awq_gemm_splitk_noalloc
    assert lib.awq_gemm_splitk_noalloc_max_bytes() == 32 << 20
    assert f(P, P2, P3, P4, P5, 64, 4096, 4096, 5, 128, NUL) == UNSUP
    assert f(P, P2, P3, P4, P5, 64, 4096, 4096, 4, 96, NUL) == UNSUP
    assert f(P, P2, P3, P4, P5, -1, 4096, 4096, 4, 128, NUL) == SHAPE
    assert f(P, P2, P3, P4, P5, 64, 4096, 4000, 4, 128, NUL) == SHAPE
    assert f(NUL, P2, P3, P4, P5, 64, 4096, 4096, 4, 128, NUL) == NULL
    assert f(P, P2, P3, P4, MIS, 64, 4096, 4096, 4, 128, NUL) == ALIGN
    assert f(NUL, NUL, NUL, NUL, NUL, 0, 4096, 4096, 4, 128, NUL) == OK     # empty: nothing launched


def test_scale_activations_validation(lib):
    assert lib.awq_scale_activations(P, P2, P3, 4, 100, NUL) == SHAPE
    assert lib.awq_scale_activations(P, P2, P3, -1, 128, NUL) == SHAPE
    assert lib.awq_scale_activations(P, NUL, P3, 4, 128, NUL) == NULL
    assert lib.awq_scale_activations(P, P2, MIS, 4, 128, NUL) == ALIGN
    assert lib.awq_scale_activations(NUL, NUL, NUL, 0, 128, NUL) == OK


def search(lib, W=P, X=P2, T=64, N=256, K=512, alphas=(0.0, 0.5), bits=4, gs=128, zp=1,
           s_out=P3, loss=NUL, best=NUL, ws=P4, ws_bytes=None):
    a = (ctypes.c_float * max(len(alphas), 1))(*alphas)
    n = len(alphas)
    if ws_bytes is None:
        ws_bytes = lib.awq_search_workspace_bytes(T, N, K, max(n, 1))
    return lib.awq_search_scale(W, X, T, N, K, ctypes.cast(a, ctypes.c_void_p), n, bits, gs, zp,
                                s_out, loss, best, ws, ws_bytes, NUL)


def test_search_validation(lib):
    assert search(lib, bits=2) == UNSUP
    assert search(lib, zp=2) == UNSUP
    assert search(lib, zp=0, W=NUL) == NULL
    assert search(lib, alphas=()) == UNSUP
    assert search(lib, alphas=tuple([0.5] * 65)) == UNSUP
    assert search(lib, T=8193) == UNSUP
    assert search(lib, T=0) == SHAPE
    assert search(lib, K=130) == SHAPE
    assert search(lib, T=8192, K=262144) == SHAPE      # T * K reaches 2^31
    assert search(lib, W=NUL) == NULL
    assert search(lib, s_out=MIS) == ALIGN
    assert search(lib, loss=MIS) == ALIGN
    # below the fused path's size: no path fits (between it and the default
    # size the fused path runs, which needs a GPU)
    least = lib.awq_search_workspace_bytes_fused(64, 256, 512, 2)
    assert 0 < least < lib.awq_search_workspace_bytes(64, 256, 512, 2)
    assert search(lib, ws_bytes=least - 1) == WS


def shared(lib, Ws=(P, P2, P3), Ns=(64, 32, 32), n=None, X=P4, T=64, K=512, alphas=(0.0, 0.5),
           bits=4, gs=128, zp=1, s_out=P5, loss=NUL, best=NUL, ws=P, ws_bytes=None):
    n = (3 if Ws is None else len(Ws)) if n is None else n
    if ws_bytes is None:
        ws_bytes = lib.awq_search_workspace_bytes(T, max(1, sum(Ns or (1,))), K, max(1, len(alphas)))
    wp = (ctypes.c_void_p * max(1, len(Ws)))(*[w.value for w in Ws]) if Ws is not None else None
    npt = (ctypes.c_int * max(1, len(Ns)))(*Ns) if Ns is not None else None
    a = (ctypes.c_float * max(1, len(alphas)))(*alphas)
    return lib.awq_search_scale_shared(ctypes.cast(wp, ctypes.c_void_p) if wp is not None else NUL,
                                       ctypes.cast(npt, ctypes.c_void_p) if npt is not None else NUL,
                                       n, X, T, K, ctypes.cast(a, ctypes.c_void_p), len(alphas), bits,
                                       gs, zp, s_out, loss, best, ws, ws_bytes, NUL)


def test_search_shared_validation(lib):
    assert shared(lib, n=0) == UNSUP
    assert shared(lib, Ws=tuple([P] * 9), Ns=tuple([16] * 9)) == UNSUP
    assert shared(lib, Ws=None) == NULL
    assert shared(lib, Ns=None) == NULL
    assert shared(lib, Ws=(P, NUL, P3)) == NULL
    assert shared(lib, Ws=(P, MIS, P3)) == ALIGN
    assert shared(lib, Ns=(64, 0, 32)) == SHAPE
    assert shared(lib, Ns=(64, -5, 32)) == SHAPE
    assert shared(lib, K=130) == SHAPE
    assert shared(lib, T=8192, K=262144) == SHAPE
    assert shared(lib, T=0) == SHAPE
    assert shared(lib, T=8193) == UNSUP
    assert shared(lib, alphas=()) == UNSUP
    assert shared(lib, bits=5) == UNSUP
    assert shared(lib, X=NUL) == NULL
    assert shared(lib, s_out=MIS) == ALIGN
    least = lib.awq_search_workspace_bytes_fused(64, 128, 512, 2)
    assert shared(lib, ws_bytes=least - 1) == WS


def test_binding_refuses_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setenv("AWQ_MI355X_LIB", str(tmp_path / "nope.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(B.AwqError):
        B.load_library()
