"""ctypes binding of libawq.so (C ABI in include/awq.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  Tensors are torch tensors on the GPU; the binding checks dtype,
device, shape and contiguity, allocates outputs with torch and passes raw
device pointers and the current HIP stream.  A missing library raises
``AwqError`` on first use; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libawq.so"

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size_t = ctypes.c_size_t

# (name, restype, argtypes) for every exported symbol of include/awq.h
SIGNATURES = [
    ("awq_status_str", ctypes.c_char_p, [_c_int]),
    ("awq_pack_format_version", _c_int, []),
    ("awq_packed_words_per_row", _c_size_t, [_c_int, _c_int]),
    ("awq_packed_words", _c_size_t, [_c_int, _c_int, _c_int]),
    ("awq_quantize_pack", _c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    ("awq_scale_activations", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_void_p]),
    ("awq_search_workspace_bytes", _c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    ("awq_search_workspace_bytes_fused", _c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    ("awq_search_scale", _c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_int,
                                  _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_size_t, _c_void_p]),
    ("awq_search_scale_shared", _c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_int, _c_int,
                                         _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    ("awq_search_mlp_workspace_bytes", _c_size_t, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    ("awq_search_scale_mlp", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                                      _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                      _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    ("awq_gemv", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                          _c_int, _c_int, _c_int, _c_void_p]),
    ("awq_gemm", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                          _c_int, _c_int, _c_int, _c_void_p]),
    ("awq_dequantize", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                                _c_int, _c_void_p]),
    ("awq_gemv_scaled", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p]),
    ("awq_gemv_gate_up", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                  _c_int, _c_void_p]),
    ("awq_gemm_splitk_workspace_bytes", _c_size_t, [_c_int, _c_int, _c_int]),
    ("awq_gemm_splitk", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_size_t, _c_void_p]),
    ("awq_gemm_scaled", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_size_t,
                                 _c_void_p]),
    ("awq_gemm_splitk_noalloc_max_bytes", _c_size_t, []),
    ("awq_gemm_splitk_noalloc", _c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p]),
]

STATUS = {0: "AWQ_OK", 1: "AWQ_ERR_NULL", 2: "AWQ_ERR_SHAPE", 3: "AWQ_ERR_UNSUPPORTED",
          4: "AWQ_ERR_ALIGN", 5: "AWQ_ERR_WORKSPACE", 6: "AWQ_ERR_HIP"}

GROUP_SIZE = 128


class AwqError(RuntimeError):
    """A non-zero status from the library, or the library is missing."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


_lib = None


def library_path() -> str:
    return os.environ.get("AWQ_MI355X_LIB", os.path.join(_HERE, "lib", LIB_NAME))


def load_library():
    """Load libawq.so once; raise AwqError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise AwqError(f"HIP library not built: {path} is missing "
                       "(run __graft_entry__.build() or python -m "
                       "weight_only_quantization_pack_amd.build)")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        name = STATUS.get(status, str(status))
        raise AwqError(f"{what} failed: {name}", status)


def _torch():
    import torch
    return torch


def _stream_ptr(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pack_format_version() -> int:
    return int(load_library().awq_pack_format_version())


def packed_words_per_row(K: int, bits: int) -> int:
    return int(load_library().awq_packed_words_per_row(K, bits))


def packed_words(N: int, K: int, bits: int) -> int:
    """uint32 words of a packed N x K matrix (format 3: rows padded to 16)."""
    return int(load_library().awq_packed_words(N, K, bits))


def quantize_pack(W, s=None, bits: int = 4, group_size: int = GROUP_SIZE,
                  zero_point: bool = True, out=None):
    """Quantize fp16 W [N][K] (times s [K] if given) and pack.

    Returns (qweight int32 [packed_words(N, K, bits)], scales fp16
    [ceil(N/16)][G][16], zeros fp16 [ceil(N/16)][G][16]) in packed format 3.
    """
    torch = _torch()
    lib = load_library()
    N, K = W.shape
    _need(W, torch.float16, (N, K), "W")
    if s is not None:
        _need(s, torch.float32, (K,), "s")
    G = K // group_size if group_size > 0 else 0
    if out is None:
        words = int(lib.awq_packed_words(N, K, bits))
        qweight = torch.empty((words,), dtype=torch.int32, device=W.device)
        NB = (N + 15) // 16
        scales = torch.empty((NB, G, 16), dtype=torch.float16, device=W.device)
        zeros = torch.empty((NB, G, 16), dtype=torch.float16, device=W.device)
    else:
        qweight, scales, zeros = out
    st = lib.awq_quantize_pack(_ptr(W), _ptr(s), N, K, bits, group_size, int(zero_point),
                               _ptr(qweight), _ptr(scales), _ptr(zeros), _stream_ptr(W))
    _check(st, "awq_quantize_pack")
    return qweight, scales, zeros


def fake_quantize(qweight, scales, zeros, N: int, K: int, bits: int = 4, group_size: int = GROUP_SIZE,
                  out=None):
    """w_hat fp16 [N][K] = fp16((q - z) * D) from the packed layer (awq_dequantize)."""
    torch = _torch()
    lib = load_library()
    _need_layer(qweight, scales, zeros, N, K, bits, group_size)
    if out is None:
        out = torch.empty((N, K), dtype=torch.float16, device=qweight.device)
    else:
        _need(out, torch.float16, (N, K), "out")
    st = lib.awq_dequantize(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(out), N, K, bits,
                            group_size, _stream_ptr(qweight))
    _check(st, "awq_dequantize")
    return out


def scale_activations(x, s, out=None):
    """x' = fp16(x / s) per input channel."""
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    _need(x, torch.float16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    if out is None:
        out = torch.empty_like(x)
    st = lib.awq_scale_activations(_ptr(x), _ptr(s), _ptr(out), M, K, _stream_ptr(x))
    _check(st, "awq_scale_activations")
    return out


def search_workspace_bytes(T: int, N: int, K: int, n_alpha: int, fused: bool = True) -> int:
    """Workspace of the search's fused path (the default: the loss kernel forms
    W - w_hat / s in registers), or (fused=False) the larger one with which the
    search writes those differences out per chunk of alphas and runs a loss GEMM."""
    lib = load_library()
    f = lib.awq_search_workspace_bytes_fused if fused else lib.awq_search_workspace_bytes
    return int(f(T, N, K, n_alpha))


def search_scale(W, X_cal, alphas, bits: int = 4, group_size: int = GROUP_SIZE,
                 zero_point: bool = True, workspace=None, fused: bool = True):
    """AWQ alpha-grid search.  Returns (s fp32 [K], loss fp32 [n_alpha], best int32 [1]).
    The path follows the workspace size (awq_search_workspace_bytes[_fused]);
    without a workspace, the one of the path `fused` names is allocated."""
    torch = _torch()
    lib = load_library()
    N, K = W.shape
    T = X_cal.shape[0]
    _need(W, torch.float16, (N, K), "W")
    _need(X_cal, torch.float16, (T, K), "X_cal")
    a = (ctypes.c_float * len(alphas))(*[float(v) for v in alphas])
    n_alpha = len(alphas)
    need = search_workspace_bytes(T, N, K, n_alpha, fused)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=W.device)
    s_out = torch.empty(K, dtype=torch.float32, device=W.device)
    loss = torch.empty(max(n_alpha, 1), dtype=torch.float32, device=W.device)
    best = torch.empty(1, dtype=torch.int32, device=W.device)
    st = lib.awq_search_scale(_ptr(W), _ptr(X_cal), T, N, K, ctypes.cast(a, _c_void_p), n_alpha,
                              bits, group_size, int(zero_point), _ptr(s_out), _ptr(loss),
                              _ptr(best), _ptr(workspace), workspace.numel(), _stream_ptr(W))
    _check(st, "awq_search_scale")
    return s_out, loss[:n_alpha], best


def search_mlp_workspace_bytes(T: int, K: int, I: int, K_out: int, n_alpha: int) -> int:
    return int(load_library().awq_search_mlp_workspace_bytes(T, K, I, K_out, n_alpha))


def search_scale_mlp(W_gate, W_up, W_down, X_cal, alphas, bits: int = 4, group_size: int = GROUP_SIZE,
                     zero_point: bool = True, workspace=None):
    """The gate/up pair's shared scale searched on the MLP block's output
    (awq_search_scale_mlp).  W_gate, W_up fp16 [I][K], W_down fp16 [K_out][I],
    X_cal fp16 [T][K].  Returns (s fp32 [K], loss fp32 [n_alpha], best int32 [1])."""
    torch = _torch()
    lib = load_library()
    I, K = W_gate.shape
    K_out = W_down.shape[0]
    T = X_cal.shape[0]
    _need(W_gate, torch.float16, (I, K), "W_gate")
    _need(W_up, torch.float16, (I, K), "W_up")
    _need(W_down, torch.float16, (K_out, I), "W_down")
    _need(X_cal, torch.float16, (T, K), "X_cal")
    n_alpha = len(alphas)
    a = (ctypes.c_float * n_alpha)(*[float(v) for v in alphas])
    need = search_mlp_workspace_bytes(T, K, I, K_out, n_alpha)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=W_gate.device)
    s_out = torch.empty(K, dtype=torch.float32, device=W_gate.device)
    loss = torch.empty(max(n_alpha, 1), dtype=torch.float32, device=W_gate.device)
    best = torch.empty(1, dtype=torch.int32, device=W_gate.device)
    st = lib.awq_search_scale_mlp(_ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(X_cal), T, K, I, K_out,
                                  ctypes.cast(a, _c_void_p), n_alpha, bits, group_size, int(zero_point),
                                  _ptr(s_out), _ptr(loss), _ptr(best), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream_ptr(W_gate))
    _check(st, "awq_search_scale_mlp")
    return s_out, loss[:n_alpha], best


def _need_layer(qweight, scales, zeros, N, K, bits, group_size, what=""):
    torch = _torch()
    words = int(load_library().awq_packed_words(N, K, bits))
    _need(qweight, torch.int32, (words,), what + "qweight")
    G = K // group_size if group_size > 0 else 0
    NB = (N + 15) // 16
    _need(scales, torch.float16, (NB, G, 16), what + "scales")
    _need(zeros, torch.float16, (NB, G, 16), what + "zeros")


def search_scale_shared(Ws, X_cal, alphas, bits: int = 4, group_size: int = GROUP_SIZE,
                        zero_point: bool = True, workspace=None, fused: bool = True):
    """One s for several layers reading X_cal (awq_search_scale_shared): the
    layers' rows together form the searched layer.  Returns (s fp32 [K],
    losses fp32 [n_alpha], best int32 [1]) as search_scale (workspace and
    fused as there)."""
    torch = _torch()
    lib = load_library()
    Ws = list(Ws)
    if not Ws:
        raise ValueError("Ws must hold at least one layer")
    T, K = X_cal.shape
    _need(X_cal, torch.float16, (T, K), "X_cal")
    for i, W in enumerate(Ws):
        _need(W, torch.float16, (W.shape[0], K), f"Ws[{i}]")
    n = len(Ws)
    ptrs = (_c_void_p * n)(*[W.data_ptr() for W in Ws])
    Ns = (ctypes.c_int * n)(*[int(W.shape[0]) for W in Ws])
    a = (ctypes.c_float * len(alphas))(*[float(v) for v in alphas])
    n_alpha = len(alphas)
    need = search_workspace_bytes(T, sum(Ns), K, n_alpha, fused)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X_cal.device)
    s_out = torch.empty(K, dtype=torch.float32, device=X_cal.device)
    loss = torch.empty(max(n_alpha, 1), dtype=torch.float32, device=X_cal.device)
    best = torch.empty(1, dtype=torch.int32, device=X_cal.device)
    st = lib.awq_search_scale_shared(ctypes.cast(ptrs, _c_void_p), ctypes.cast(Ns, _c_void_p), n,
                                     _ptr(X_cal), T, K, ctypes.cast(a, _c_void_p), n_alpha, bits,
                                     group_size, int(zero_point), _ptr(s_out), _ptr(loss), _ptr(best),
                                     _ptr(workspace), workspace.numel(), _stream_ptr(X_cal))
    _check(st, "awq_search_scale_shared")
    return s_out, loss[:n_alpha], best


def _matmul(fn_name, x, qweight, scales, zeros, N, bits, group_size, out, workspace=None):
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    _need(x, torch.float16, (M, K), "x")
    _need_layer(qweight, scales, zeros, N, K, bits, group_size)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, (M, N), "out")
    if fn_name == "awq_gemm_splitk":
        st = lib.awq_gemm_splitk(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(out),
                                 M, N, K, bits, group_size, _ptr(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _stream_ptr(x))
    else:
        st = getattr(lib, fn_name)(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(out),
                                   M, N, K, bits, group_size, _stream_ptr(x))
    _check(st, fn_name)
    return out


def _gemm_scaled(x, inv_s, qweight, scales, zeros, N, bits, group_size, out, split_k, workspace):
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    _need(x, torch.float16, (M, K), "x")
    _need(inv_s, torch.float32, (K,), "inv_s")
    _need_layer(qweight, scales, zeros, N, K, bits, group_size)
    out = _out(out, M, N, x.device)
    need = gemm_splitk_workspace_bytes(M, N, K) if split_k else 0
    if need == 0:
        workspace = None
    elif workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    st = lib.awq_gemm_scaled(_ptr(x), _ptr(inv_s), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(out),
                             M, N, K, bits, group_size, _ptr(workspace),
                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                             _stream_ptr(x))
    _check(st, "awq_gemm_scaled")
    return out


def gemm_splitk_noalloc(x, qweight, scales, zeros, N: int, bits: int = 4,
                        group_size: int = GROUP_SIZE, out=None):
    """awq_gemm_splitk_noalloc: the split-K prefill product with its fp32
    partials in the library's fixed per-GPU array (the call allocates no device
    memory; `out` is allocated here only when not given).  Calls overlapping on
    one GPU race on that array."""
    return _matmul("awq_gemm_splitk_noalloc", x, qweight, scales, zeros, N, bits, group_size, out)


def gemm_splitk_noalloc_max_bytes() -> int:
    """Size of the fixed partial-sum array of awq_gemm_splitk_noalloc."""
    return int(load_library().awq_gemm_splitk_noalloc_max_bytes())


def gemv(x, qweight, scales, zeros, N: int, bits: int = 4, group_size: int = GROUP_SIZE, out=None,
         inv_s=None):
    """Decode product y = x . w_hat^T for 1 <= M <= 16 rows of x; N output columns.

    inv_s (fp32 [K] device tensor, the reciprocal of the AWQ scale) folds the
    activation scale into the load: y = fp16(x * inv_s) . w_hat^T through
    awq_gemv_scaled."""
    if inv_s is None:
        return _matmul("awq_gemv", x, qweight, scales, zeros, N, bits, group_size, out)
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    _need(x, torch.float16, (M, K), "x")
    _need(inv_s, torch.float32, (K,), "inv_s")
    _need_layer(qweight, scales, zeros, N, K, bits, group_size)
    out = _out(out, M, N, x.device)
    st = lib.awq_gemv_scaled(_ptr(x), _ptr(inv_s), _ptr(qweight), _ptr(scales), _ptr(zeros),
                             _ptr(out), M, N, K, bits, group_size, _stream_ptr(x))
    _check(st, "awq_gemv_scaled")
    return out


def gemv_gate_up(x, gate, up, N: int, bits: int = 4, group_size: int = GROUP_SIZE, inv_s=None,
                 out=None):
    """Gate/up half of a fused MLP in one launch: h = SiLU(x' . w_gate^T) * (x' . w_up^T).

    gate, up: (qweight, scales, zeros) of two N x K layers; x' = fp16(x * inv_s)
    when inv_s (fp32 [K]) is given, else x.  h fp16 [M][N] (awq_gemv_gate_up)."""
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    _need(x, torch.float16, (M, K), "x")
    if inv_s is not None:
        _need(inv_s, torch.float32, (K,), "inv_s")
    _need_layer(*gate, N, K, bits, group_size, "gate ")
    _need_layer(*up, N, K, bits, group_size, "up ")
    out = _out(out, M, N, x.device)
    st = lib.awq_gemv_gate_up(_ptr(x), _ptr(inv_s), _ptr(gate[0]), _ptr(gate[1]), _ptr(gate[2]),
                              _ptr(up[0]), _ptr(up[1]), _ptr(up[2]), _ptr(out), M, N, K, bits,
                              group_size, _stream_ptr(x))
    _check(st, "awq_gemv_gate_up")
    return out


def _out(out, M, N, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=torch.float16, device=device)
    _need(out, torch.float16, (M, N), "out")
    return out


def gemm_splitk_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes awq_gemm_splitk needs for this shape (0: no split)."""
    return int(load_library().awq_gemm_splitk_workspace_bytes(M, N, K))


def gemm(x, qweight, scales, zeros, N: int, bits: int = 4, group_size: int = GROUP_SIZE, out=None,
         split_k: bool = True, workspace=None, inv_s=None):
    """Prefill product y = x . w_hat^T for any M >= 1 rows of x (bits 4 or 3); N output columns.

    With split_k (default) shapes with few output tiles run through
    awq_gemm_splitk; its fp32 workspace is `workspace` (a device tensor of at
    least gemm_splitk_workspace_bytes bytes) or allocated here.  split_k=False
    always calls awq_gemm.  inv_s (fp32 [K] device tensor, the reciprocal of
    the AWQ scale) folds the activation scale into the product through
    awq_gemm_scaled: y = fp16(x * inv_s) . w_hat^T.
    """
    if inv_s is not None:
        return _gemm_scaled(x, inv_s, qweight, scales, zeros, N, bits, group_size, out, split_k,
                            workspace)
    if split_k and x.dim() == 2:
        need = gemm_splitk_workspace_bytes(x.shape[0], N, x.shape[1])
        if need > 0:
            if workspace is None:
                workspace = _torch().empty(need, dtype=_torch().uint8, device=x.device)
            return _matmul("awq_gemm_splitk", x, qweight, scales, zeros, N, bits, group_size, out,
                           workspace)
    return _matmul("awq_gemm", x, qweight, scales, zeros, N, bits, group_size, out)
