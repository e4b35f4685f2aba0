"""Fused transformer feed-forward kernels for AMD MI355X (gfx950).

Thin Python binding of the C-ABI library ``libfmlp.so`` (declared in
``include/fmlp.h``).  It only marshals arguments: it checks tensor dtypes and
devices, flattens leading dims (M = batch * seq), allocates outputs and
workspaces with torch, and passes raw device pointers plus the current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind: if the library is not built, every call
raises.

    fmlp_linear(x, W, b=None, act="none")          y = act(x W^T + b)
    fmlp_mlp2(x, W1, b1, W2, b2, act)               y = act(x W1^T + b1) W2^T + b2
    fmlp_geglu(x, Wg, Wu, Wd)                       y = (gelu_tanh(x Wg^T) * x Wu^T) Wd^T
    fmlp_glu(x, Wg, Wu, Wd, gate_act)               y = (gate_act(x Wg^T) * x Wu^T) Wd^T
    fmlp_glu_noalloc(x, Wg, Wu, Wd, gate_act)       the same with the library's own scratch array
    fmlp_moe_geglu(x, expert_ids, gate_w, Wg, Wu, Wd)
                                                    y[t] = sum_j w[t,j] geglu_{e[t,j]}(x[t])
    fmlp_moe_glu(x, expert_ids, gate_w, Wg, Wu, Wd, gate_act)
    fmlp_linear_w8(x, Wq, s, b, act)               the same forms with FP8 E4M3 weights and a
    fmlp_mlp2_w8(x, W1q, s1, b1, W2q, s2, b2, act)  scale per output row, W = s[:, None] * e4m3(Wq);
    fmlp_glu_w8(x, Wgq, sg, Wuq, su, Wdq, sd, act)  decode only (at most 16 tokens)
    fmlp_moe_route(x, Wr, top_k)                    -> (expert_ids, gate_w[, logits]): top_k of x Wr^T,
                                                       softmax over the chosen logits

    fmlp_linear_bwd(x, W, b, act, dy)               -> (dx, dW, db): gradients of fmlp_linear
    fmlp_glu_bwd(x, Wg, Wu, Wd, gate_act, dy)       -> (dx, dWg, dWu, dWd): gradients of fmlp_glu

Activations: "none", "gelu_erf", "gelu_tanh", "relu", "silu".
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

__all__ = [
    "FmlpError",
    "ACT",
    "library_path",
    "lib",
    "fmlp_linear",
    "fmlp_mlp2",
    "fmlp_geglu",
    "fmlp_glu",
    "fmlp_glu_noalloc",
    "fmlp_linear_bwd",
    "fmlp_glu_bwd",
    "bind_linear_bwd",
    "bind_glu_bwd",
    "fmlp_moe_geglu",
    "fmlp_moe_glu",
    "fmlp_moe_route",
    "fmlp_linear_w8",
    "fmlp_mlp2_w8",
    "fmlp_glu_w8",
    "bind_linear_w8",
    "bind_mlp2_w8",
    "bind_glu_w8",
    "bind_moe_route",
    "fmlp_mlp2_workspace_size",
    "fmlp_geglu_workspace_size",
    "fmlp_moe_workspace_size",
    "force_path",
    "cooperative_decode",
    "workspace_for",
    "barrier_timeouts",
    "decode_generation",
    "moe_invalid_ids",
    "BoundCall",
    "bind_mlp2",
    "bind_geglu",
    "bind_glu",
    "bind_moe_geglu",
    "bind_moe_glu",
    "bind_linear",
    "linear",
    "mlp2",
    "geglu",
    "moe_geglu",
]

ACT = {"none": 0, "gelu_erf": 1, "gelu_tanh": 2, "relu": 3, "silu": 4}
PATHS = {"auto": 0, "decode": 1, "gemm": 2, "small": 3, "fused": 4}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libfmlp.so")


class FmlpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"fmlp status {status}: {detail}")


_lib = None
_lib_lock = threading.Lock()

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libfmlp.so (built in-tree).  Raises if it is missing."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise FmlpError(-1, f"{path} is not built; run gemm_epilogue_bf16_amd.build.build() "
                                "(there is no non-HIP fallback)")
        L = ctypes.CDLL(path)
        L.fmlp_linear.argtypes = [_p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p]
        L.fmlp_mlp2.argtypes = [_p, _p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p, _sz, _p]
        L.fmlp_geglu.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _sz, _p]
        L.fmlp_glu.argtypes = [_p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _sz, _p]
        L.fmlp_moe_geglu.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, ctypes.c_int32,
                                     ctypes.c_int32, _p, _p, _sz, _p]
        L.fmlp_moe_glu.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int32,
                                   ctypes.c_int32, _p, _p, _sz, _p]
        L.fmlp_moe_route.argtypes = [_p, _p, _i64, _i64, ctypes.c_int32, ctypes.c_int32, _p, _p, _p, _p]
        L.fmlp_glu_noalloc.argtypes = [_p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p]
        L.fmlp_glu_noalloc.restype = ctypes.c_int
        L.fmlp_linear_bwd.argtypes = [_p, _p, _p, ctypes.c_int, _p, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p]
        L.fmlp_linear_bwd.restype = ctypes.c_int
        L.fmlp_glu_bwd.argtypes = [_p, _p, _p, _p, ctypes.c_int, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _sz, _p]
        L.fmlp_glu_bwd.restype = ctypes.c_int
        for f, n in (("fmlp_linear_bwd_workspace_size", 3), ("fmlp_glu_bwd_workspace_size", 3)):
            getattr(L, f).argtypes = [_i64] * n
            getattr(L, f).restype = _sz
        for f in ("fmlp_linear", "fmlp_mlp2", "fmlp_geglu", "fmlp_glu", "fmlp_moe_geglu", "fmlp_moe_glu",
                  "fmlp_moe_route", "fmlp_set_path", "fmlp_set_cooperative_decode"):
            getattr(L, f).restype = ctypes.c_int
        L.fmlp_linear_w8.argtypes = [_p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p]
        L.fmlp_mlp2_w8.argtypes = [_p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p,
                                   _sz, _p]
        L.fmlp_glu_w8.argtypes = [_p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _sz, _p]
        L.fmlp_w8_workspace_size.argtypes = [_i64, _i64]
        L.fmlp_w8_workspace_size.restype = _sz
        L.fmlp_set_path.argtypes = [ctypes.c_int]
        L.fmlp_set_cooperative_decode.argtypes = [ctypes.c_int]
        L.fmlp_mlp2_workspace_size.argtypes = [_i64, _i64, _i64, _i64]
        L.fmlp_mlp2_workspace_size.restype = _sz
        L.fmlp_geglu_workspace_size.argtypes = [_i64, _i64, _i64]
        L.fmlp_geglu_workspace_size.restype = _sz
        L.fmlp_glu_workspace_size.argtypes = [_i64, _i64, _i64]
        L.fmlp_glu_workspace_size.restype = _sz
        L.fmlp_moe_workspace_size.argtypes = [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_int32]
        L.fmlp_moe_workspace_size.restype = _sz
        L.fmlp_moe_error_offset.argtypes = []
        L.fmlp_moe_error_offset.restype = _sz
        for f in ("fmlp_decode_timeout_offset", "fmlp_decode_generation_offset"):
            getattr(L, f).argtypes = []
            getattr(L, f).restype = _sz
        L.fmlp_status_string.argtypes = [ctypes.c_int]
        L.fmlp_status_string.restype = ctypes.c_char_p
        L.fmlp_last_error.argtypes = []
        L.fmlp_last_error.restype = ctypes.c_char_p
        L.fmlp_version.argtypes = []
        L.fmlp_version.restype = ctypes.c_int
        _lib = L
        return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise FmlpError(status, f"{L.fmlp_status_string(status).decode()} -- {L.fmlp_last_error().decode()}")


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dev_tensor(name: str, t: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_ws_cache: dict = {}
_ws_lock = threading.Lock()


def workspace_for(device: torch.device, nbytes: int) -> torch.Tensor:
    """A zero-initialised workspace of at least nbytes, cached per (device,
    stream).  Its 8 KB header (barrier words) must start zeroed; calls keep it
    consistent."""
    if nbytes <= 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


@contextlib.contextmanager
def cooperative_decode():
    """The calling thread's one-launch decode calls use a cooperative launch
    (a grid that cannot be resident at once is refused instead of timing out)."""
    L = lib()
    _check(L.fmlp_set_cooperative_decode(1))
    try:
        yield
    finally:
        L.fmlp_set_cooperative_decode(0)


@contextlib.contextmanager
def force_path(path: str):
    """Force the calling thread's mlp2/glu path: "auto", "decode", "gemm", "small" (mlp2 only) or
    "fused" (the gated block in one launch, D <= 1024)."""
    L = lib()
    _check(L.fmlp_set_path(PATHS[path]))
    try:
        yield
    finally:
        L.fmlp_set_path(0)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
class BoundCall:
    """One C-ABI call with its arguments marshalled once (device pointers,
    sizes, workspace, stream).  Calling it re-enqueues the same launch with a
    single foreign call: for tight decode loops, where per-call Python
    marshalling would cost more than the kernel itself."""

    __slots__ = ("_fn", "_args", "out", "_keep")

    def __init__(self, fn, args, out, keep=()):
        self._fn = fn
        self._args = tuple(args)
        self.out = out
        self._keep = tuple(keep)   # the tensors whose pointers args hold

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            _check(st)
        return self.out


def _linear_call(x, W, b, act, out):
    _dev_tensor("x", x)
    _dev_tensor("W", W)
    if b is not None:
        _dev_tensor("b", b)
    K = x.shape[-1]
    N = W.shape[0]
    if W.dim() != 2 or W.shape[1] != K:
        raise ValueError(f"W must be [N, {K}], got {tuple(W.shape)}")
    M = x.numel() // K if K else 0
    y = out if out is not None else torch.empty(*x.shape[:-1], N, dtype=torch.bfloat16, device=x.device)
    _dev_tensor("out", y)
    return BoundCall(lib().fmlp_linear, (_ptr(x), _ptr(W), _ptr(b), ACT[act], M, K, N, _ptr(y),
                                         _stream(x.device)), y, (x, W, b))


def fmlp_linear(x, W, b=None, act: str = "none", out=None):
    """y = act(x W^T + b); x [..., K], W [N, K], b [N] or None -> y [..., N]."""
    with torch.cuda.device(x.device):
        return _linear_call(x, W, b, act, out)()


def bind_linear(x, W, b=None, act: str = "none", out=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _linear_call(x, W, b, act, out)


def fmlp_mlp2_workspace_size(M, K, H, N) -> int:
    return int(lib().fmlp_mlp2_workspace_size(M, K, H, N))


def _mlp2_call(x, W1, b1, W2, b2, act, out, workspace):
    for n, t in (("x", x), ("W1", W1), ("W2", W2)):
        _dev_tensor(n, t)
    for n, t in (("b1", b1), ("b2", b2)):
        if t is not None:
            _dev_tensor(n, t)
    K = x.shape[-1]
    H, N = W1.shape[0], W2.shape[0]
    if W1.shape[1] != K or W2.shape[1] != H:
        raise ValueError(f"shape mismatch: x[...,{K}] W1{tuple(W1.shape)} W2{tuple(W2.shape)}")
    M = x.numel() // K
    y = out if out is not None else torch.empty(*x.shape[:-1], N, dtype=torch.bfloat16, device=x.device)
    L = lib()
    need = int(L.fmlp_mlp2_workspace_size(M, K, H, N))
    ws = workspace if workspace is not None else workspace_for(x.device, need)
    return BoundCall(L.fmlp_mlp2, (_ptr(x), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), ACT[act], M, K, H,
                                   N, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(x.device)), y, (x, W1, b1, W2, b2, ws))


def fmlp_mlp2(x, W1, b1, W2, b2, act: str = "gelu_erf", out=None, workspace=None):
    """y = act(x W1^T + b1) W2^T + b2; W1 [H, K], W2 [N, H]; biases may be None."""
    with torch.cuda.device(x.device):
        return _mlp2_call(x, W1, b1, W2, b2, act, out, workspace)()


def bind_mlp2(x, W1, b1, W2, b2, act: str = "gelu_erf", out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _mlp2_call(x, W1, b1, W2, b2, act, out, workspace)


def fmlp_geglu_workspace_size(M, D, H) -> int:
    return int(lib().fmlp_geglu_workspace_size(M, D, H))


def _geglu_call(x, Wg, Wu, Wd, out, workspace, gate_act=None):
    for n, t in (("x", x), ("Wg", Wg), ("Wu", Wu), ("Wd", Wd)):
        _dev_tensor(n, t)
    D = x.shape[-1]
    H = Wg.shape[0]
    if Wg.shape != (H, D) or Wu.shape != (H, D) or Wd.shape != (D, H):
        raise ValueError(f"shape mismatch: x[...,{D}] Wg{tuple(Wg.shape)} Wu{tuple(Wu.shape)} Wd{tuple(Wd.shape)}")
    M = x.numel() // D
    y = out if out is not None else torch.empty_like(x)
    L = lib()
    need = int(L.fmlp_geglu_workspace_size(M, D, H))
    ws = workspace if workspace is not None else workspace_for(x.device, need)
    if gate_act is None:
        return BoundCall(L.fmlp_geglu, (_ptr(x), _ptr(Wg), _ptr(Wu), _ptr(Wd), M, D, H, _ptr(y), _ptr(ws),
                                        ws.numel(), _stream(x.device)), y, (x, Wg, Wu, Wd, ws))
    return BoundCall(L.fmlp_glu, (_ptr(x), _ptr(Wg), _ptr(Wu), _ptr(Wd), ACT[gate_act], M, D, H, _ptr(y),
                                  _ptr(ws), ws.numel(), _stream(x.device)), y, (x, Wg, Wu, Wd, ws))


def fmlp_geglu(x, Wg, Wu, Wd, out=None, workspace=None):
    """y = (gelu_tanh(x Wg^T) * (x Wu^T)) Wd^T; Wg, Wu [H, D], Wd [D, H]."""
    with torch.cuda.device(x.device):
        return _geglu_call(x, Wg, Wu, Wd, out, workspace)()


def bind_geglu(x, Wg, Wu, Wd, out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _geglu_call(x, Wg, Wu, Wd, out, workspace)


def fmlp_glu(x, Wg, Wu, Wd, gate_act: str = "silu", out=None, workspace=None):
    """y = (gate_act(x Wg^T) * (x Wu^T)) Wd^T; "silu" is SwiGLU, "gelu_tanh" GeGLU."""
    with torch.cuda.device(x.device):
        return _geglu_call(x, Wg, Wu, Wd, out, workspace, gate_act)()


def bind_glu(x, Wg, Wu, Wd, gate_act: str = "silu", out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _geglu_call(x, Wg, Wu, Wd, out, workspace, gate_act)


def fmlp_glu_noalloc(x, Wg, Wu, Wd, gate_act: str = "silu", out=None):
    """fmlp_glu without a workspace: the library's own fixed device array serves
    as one (for callers that cannot allocate).  Calls on one device must be
    ordered on one stream."""
    with torch.cuda.device(x.device):
        for n, t in (("x", x), ("Wg", Wg), ("Wu", Wu), ("Wd", Wd)):
            _dev_tensor(n, t)
        D = x.shape[-1]
        H = Wg.shape[0]
        if Wg.shape != (H, D) or Wu.shape != (H, D) or Wd.shape != (D, H):
            raise ValueError(f"shape mismatch: x[...,{D}] Wg{tuple(Wg.shape)} Wu{tuple(Wu.shape)} "
                             f"Wd{tuple(Wd.shape)}")
        M = x.numel() // D
        y = out if out is not None else torch.empty_like(x)
        _dev_tensor("out", y)
        _check(lib().fmlp_glu_noalloc(_ptr(x), _ptr(Wg), _ptr(Wu), _ptr(Wd), ACT[gate_act], M, D, H, _ptr(y),
                                      _stream(x.device)))
        return y


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------
def _linear_bwd_call(x, W, b, act, dy, out, workspace):
    _dev_tensor("x", x)
    _dev_tensor("W", W)
    _dev_tensor("dy", dy)
    if b is not None:
        _dev_tensor("b", b)
    K = x.shape[-1]
    N = W.shape[0]
    if W.dim() != 2 or W.shape[1] != K:
        raise ValueError(f"W must be [N, {K}], got {tuple(W.shape)}")
    M = x.numel() // K
    if dy.numel() != M * N:
        raise ValueError(f"dy must hold {M} x {N} values")
    if out is not None:
        dx, dW, db = out
    else:
        dx = torch.empty_like(x)
        dW = torch.empty_like(W)
        db = torch.empty(N, dtype=torch.bfloat16, device=x.device) if b is not None else None
    for n, t in (("dx", dx), ("dW", dW)):
        _dev_tensor(n, t)
    L = lib()
    need = int(L.fmlp_linear_bwd_workspace_size(M, K, N))
    ws = workspace if workspace is not None else workspace_for(x.device, need)
    return BoundCall(L.fmlp_linear_bwd, (_ptr(x), _ptr(W), _ptr(b), ACT[act], _ptr(dy), M, K, N, _ptr(dx), _ptr(dW),
                                         _ptr(db), _ptr(ws), 0 if ws is None else ws.numel(), _stream(x.device)),
                     (dx, dW, db), (x, W, b, dy, dx, dW, db, ws))


def fmlp_linear_bwd(x, W, b, act: str, dy, out=None, workspace=None):
    """Gradients of y = act(x W^T + b): returns (dx, dW, db) (db None without b)."""
    with torch.cuda.device(x.device):
        return _linear_bwd_call(x, W, b, act, dy, out, workspace)()


def bind_linear_bwd(x, W, b, act: str, dy, out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _linear_bwd_call(x, W, b, act, dy, out, workspace)


def _glu_bwd_call(x, Wg, Wu, Wd, gate_act, dy, out, workspace):
    for n, t in (("x", x), ("Wg", Wg), ("Wu", Wu), ("Wd", Wd), ("dy", dy)):
        _dev_tensor(n, t)
    D = x.shape[-1]
    H = Wg.shape[0]
    if Wg.shape != (H, D) or Wu.shape != (H, D) or Wd.shape != (D, H) or dy.shape != x.shape:
        raise ValueError("shape mismatch: x, dy [..., D]; Wg, Wu [H, D]; Wd [D, H]")
    M = x.numel() // D
    if out is not None:
        dx, dWg, dWu, dWd = out
    else:
        dx, dWg, dWu, dWd = torch.empty_like(x), torch.empty_like(Wg), torch.empty_like(Wu), torch.empty_like(Wd)
    L = lib()
    need = int(L.fmlp_glu_bwd_workspace_size(M, D, H))
    ws = workspace if workspace is not None else workspace_for(x.device, need)
    return BoundCall(L.fmlp_glu_bwd, (_ptr(x), _ptr(Wg), _ptr(Wu), _ptr(Wd), ACT[gate_act], _ptr(dy), M, D, H,
                                      _ptr(dx), _ptr(dWg), _ptr(dWu), _ptr(dWd), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(x.device)),
                     (dx, dWg, dWu, dWd), (x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, ws))


def fmlp_glu_bwd(x, Wg, Wu, Wd, gate_act: str, dy, out=None, workspace=None):
    """Gradients of the gated block ("gelu_tanh": GeGLU): returns (dx, dWg, dWu, dWd)."""
    with torch.cuda.device(x.device):
        return _glu_bwd_call(x, Wg, Wu, Wd, gate_act, dy, out, workspace)()


def bind_glu_bwd(x, Wg, Wu, Wd, gate_act: str, dy, out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _glu_bwd_call(x, Wg, Wu, Wd, gate_act, dy, out, workspace)


def fmlp_moe_workspace_size(T, D, H, E, top_k) -> int:
    return int(lib().fmlp_moe_workspace_size(T, D, H, E, top_k))


def _moe_call(x, expert_ids, gate_w, Wg, Wu, Wd, out, workspace, gate_act=None):
    for n, t in (("x", x), ("Wg", Wg), ("Wu", Wu), ("Wd", Wd)):
        _dev_tensor(n, t)
    _dev_tensor("expert_ids", expert_ids, torch.int32)
    _dev_tensor("gate_w", gate_w, torch.float32)
    T, D = x.shape
    E, H = Wg.shape[0], Wg.shape[1]
    k = expert_ids.shape[1]
    if Wg.shape != (E, H, D) or Wu.shape != (E, H, D) or Wd.shape != (E, D, H):
        raise ValueError("expert weight shapes must be Wg,Wu [E,H,D] and Wd [E,D,H]")
    if expert_ids.shape != (T, k) or gate_w.shape != (T, k):
        raise ValueError("routes must be [T, top_k]")
    y = out if out is not None else torch.empty_like(x)
    L = lib()
    need = int(L.fmlp_moe_workspace_size(T, D, H, E, k))
    ws = workspace if workspace is not None else workspace_for(x.device, need)
    keep = (x, expert_ids, gate_w, Wg, Wu, Wd, ws)
    if gate_act is None:
        return BoundCall(L.fmlp_moe_geglu, (_ptr(x), _ptr(expert_ids), _ptr(gate_w), _ptr(Wg), _ptr(Wu),
                                            _ptr(Wd), T, D, H, E, k, _ptr(y), _ptr(ws), ws.numel(),
                                            _stream(x.device)), y, keep)
    return BoundCall(L.fmlp_moe_glu, (_ptr(x), _ptr(expert_ids), _ptr(gate_w), _ptr(Wg), _ptr(Wu), _ptr(Wd),
                                      ACT[gate_act], T, D, H, E, k, _ptr(y), _ptr(ws), ws.numel(),
                                      _stream(x.device)), y, keep)


def fmlp_moe_geglu(x, expert_ids, gate_w, Wg, Wu, Wd, out=None, workspace=None):
    """Top-k MoE of GeGLU experts.  x [T, D]; expert_ids int32 [T, k];
    gate_w fp32 [T, k]; Wg, Wu [E, H, D]; Wd [E, D, H]."""
    with torch.cuda.device(x.device):
        return _moe_call(x, expert_ids, gate_w, Wg, Wu, Wd, out, workspace)()


def bind_moe_geglu(x, expert_ids, gate_w, Wg, Wu, Wd, out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _moe_call(x, expert_ids, gate_w, Wg, Wu, Wd, out, workspace)


def fmlp_moe_glu(x, expert_ids, gate_w, Wg, Wu, Wd, gate_act: str = "silu", out=None, workspace=None):
    """Top-k MoE of gated experts with the given gate activation ("silu": SwiGLU)."""
    with torch.cuda.device(x.device):
        return _moe_call(x, expert_ids, gate_w, Wg, Wu, Wd, out, workspace, gate_act)()


def bind_moe_glu(x, expert_ids, gate_w, Wg, Wu, Wd, gate_act: str = "silu", out=None,
                 workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _moe_call(x, expert_ids, gate_w, Wg, Wu, Wd, out, workspace, gate_act)


def _route_call(x, Wr, top_k, with_logits, out):
    _dev_tensor("x", x)
    _dev_tensor("Wr", Wr)
    T, D = x.shape
    E = Wr.shape[0]
    if Wr.shape != (E, D):
        raise ValueError(f"Wr must be [E, {D}], got {tuple(Wr.shape)}")
    if out is not None:
        ids, gw = out[0], out[1]
        lg = out[2] if with_logits else None
    else:
        ids = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
        gw = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
        lg = torch.empty(T, E, dtype=torch.float32, device=x.device) if with_logits else None
    _dev_tensor("expert_ids", ids, torch.int32)
    _dev_tensor("gate_w", gw, torch.float32)
    if lg is not None:
        _dev_tensor("logits", lg, torch.float32)
    res = (ids, gw, lg) if with_logits else (ids, gw)
    return BoundCall(lib().fmlp_moe_route, (_ptr(x), _ptr(Wr), T, D, E, top_k, _ptr(ids), _ptr(gw), _ptr(lg),
                                           _stream(x.device)), res, (x, Wr, ids, gw, lg))


def fmlp_moe_route(x, Wr, top_k: int, with_logits: bool = False, out=None):
    """Routes on the device: x [T, D], Wr [E, D] -> expert_ids int32 [T, top_k],
    gate_w fp32 [T, top_k] (and logits fp32 [T, E] with with_logits)."""
    with torch.cuda.device(x.device):
        return _route_call(x, Wr, top_k, with_logits, out)()


def bind_moe_route(x, Wr, top_k: int, with_logits: bool = False, out=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _route_call(x, Wr, top_k, with_logits, out)


# ---------------------------------------------------------------------------
# diagnostics (read after a sync)
# ---------------------------------------------------------------------------
def _ws_word(workspace: torch.Tensor, off: int) -> int:
    return int(workspace[off:off + 4].view(torch.int32).item()) & 0xFFFFFFFF


def barrier_timeouts(workspace: torch.Tensor) -> int:
    """Times the persistent decode kernel's device-wide barrier gave up waiting
    (cumulative over the calls on this workspace)."""
    return _ws_word(workspace, int(lib().fmlp_decode_timeout_offset()))


def decode_generation(workspace: torch.Tensor) -> int:
    """The workspace's decode generation: advanced by one per one-launch decode call."""
    return _ws_word(workspace, int(lib().fmlp_decode_generation_offset()))


def moe_invalid_ids(workspace: torch.Tensor) -> int:
    """Invalid expert ids seen by the last fmlp_moe_geglu call on this workspace."""
    off = int(lib().fmlp_moe_error_offset())
    return int(workspace[off:off + 4].view(torch.int32).item())


linear = fmlp_linear
mlp2 = fmlp_mlp2
geglu = fmlp_geglu
moe_geglu = fmlp_moe_geglu


# ---------------------------------------------------------------------------
# FP8 (E4M3) weights, decode
# ---------------------------------------------------------------------------
def _w8_codes(name: str, t: torch.Tensor) -> torch.Tensor:
    """FP8 weights as raw E4M3 codes: a uint8 tensor, or a float8_e4m3fn one (same bytes)."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return _dev_tensor(name, t, torch.uint8)


def _w8_scale(name: str, t: torch.Tensor, rows: int) -> torch.Tensor:
    _dev_tensor(name, t, torch.float32)
    if t.shape != (rows,):
        raise ValueError(f"{name} must be [{rows}] fp32, got {tuple(t.shape)}")
    return t


def _linear_w8_call(x, Wq, s, b, act, out):
    _dev_tensor("x", x)
    Wq = _w8_codes("Wq", Wq)
    if b is not None:
        _dev_tensor("b", b)
    K = x.shape[-1]
    N = Wq.shape[0]
    if Wq.dim() != 2 or Wq.shape[1] != K:
        raise ValueError(f"Wq must be [N, {K}], got {tuple(Wq.shape)}")
    _w8_scale("w_scale", s, N)
    M = x.numel() // K if K else 0
    y = out if out is not None else torch.empty(*x.shape[:-1], N, dtype=torch.bfloat16, device=x.device)
    _dev_tensor("out", y)
    return BoundCall(lib().fmlp_linear_w8, (_ptr(x), _ptr(Wq), _ptr(s), _ptr(b), ACT[act], M, K, N, _ptr(y),
                                            _stream(x.device)), y, (x, Wq, s, b))


def fmlp_linear_w8(x, Wq, w_scale, b=None, act: str = "none", out=None):
    """y = act(x W^T + b), W = w_scale[:, None] * e4m3(Wq); x [..., K] with at most 16 rows."""
    with torch.cuda.device(x.device):
        return _linear_w8_call(x, Wq, w_scale, b, act, out)()


def bind_linear_w8(x, Wq, w_scale, b=None, act: str = "none", out=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _linear_w8_call(x, Wq, w_scale, b, act, out)


def _mlp2_w8_call(x, W1q, s1, b1, W2q, s2, b2, act, out, workspace):
    _dev_tensor("x", x)
    W1q, W2q = _w8_codes("W1q", W1q), _w8_codes("W2q", W2q)
    for n, t in (("b1", b1), ("b2", b2)):
        if t is not None:
            _dev_tensor(n, t)
    K = x.shape[-1]
    H, N = W1q.shape[0], W2q.shape[0]
    if W1q.shape[1] != K or W2q.shape[1] != H:
        raise ValueError(f"shape mismatch: x[...,{K}] W1q{tuple(W1q.shape)} W2q{tuple(W2q.shape)}")
    _w8_scale("s1", s1, H)
    _w8_scale("s2", s2, N)
    M = x.numel() // K
    y = out if out is not None else torch.empty(*x.shape[:-1], N, dtype=torch.bfloat16, device=x.device)
    L = lib()
    ws = workspace if workspace is not None else workspace_for(x.device, int(L.fmlp_w8_workspace_size(M, H)))
    return BoundCall(L.fmlp_mlp2_w8, (_ptr(x), _ptr(W1q), _ptr(s1), _ptr(b1), _ptr(W2q), _ptr(s2), _ptr(b2),
                                      ACT[act], M, K, H, N, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                      _stream(x.device)), y, (x, W1q, s1, b1, W2q, s2, b2, ws))


def fmlp_mlp2_w8(x, W1q, s1, b1, W2q, s2, b2, act: str = "gelu_erf", out=None, workspace=None):
    """fmlp_mlp2 with FP8 weights W1 = s1 * e4m3(W1q) [H, K], W2 = s2 * e4m3(W2q) [N, H]."""
    with torch.cuda.device(x.device):
        return _mlp2_w8_call(x, W1q, s1, b1, W2q, s2, b2, act, out, workspace)()


def bind_mlp2_w8(x, W1q, s1, b1, W2q, s2, b2, act: str = "gelu_erf", out=None, workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _mlp2_w8_call(x, W1q, s1, b1, W2q, s2, b2, act, out, workspace)


def _glu_w8_call(x, Wgq, sg, Wuq, su, Wdq, sd, gate_act, out, workspace):
    _dev_tensor("x", x)
    Wgq, Wuq, Wdq = _w8_codes("Wgq", Wgq), _w8_codes("Wuq", Wuq), _w8_codes("Wdq", Wdq)
    D = x.shape[-1]
    H = Wgq.shape[0]
    if Wgq.shape != (H, D) or Wuq.shape != (H, D) or Wdq.shape != (D, H):
        raise ValueError(f"shape mismatch: x[...,{D}] Wgq{tuple(Wgq.shape)} Wuq{tuple(Wuq.shape)} "
                         f"Wdq{tuple(Wdq.shape)}")
    _w8_scale("sg", sg, H)
    _w8_scale("su", su, H)
    _w8_scale("sd", sd, D)
    M = x.numel() // D
    y = out if out is not None else torch.empty_like(x)
    L = lib()
    ws = workspace if workspace is not None else workspace_for(x.device, int(L.fmlp_w8_workspace_size(M, H)))
    return BoundCall(L.fmlp_glu_w8, (_ptr(x), _ptr(Wgq), _ptr(sg), _ptr(Wuq), _ptr(su), _ptr(Wdq), _ptr(sd),
                                     ACT[gate_act], M, D, H, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(x.device)), y, (x, Wgq, sg, Wuq, su, Wdq, sd, ws))


def fmlp_glu_w8(x, Wgq, sg, Wuq, su, Wdq, sd, gate_act: str = "gelu_tanh", out=None, workspace=None):
    """fmlp_glu with FP8 weights: Wg = sg * e4m3(Wgq), Wu = su * e4m3(Wuq) [H, D], Wd = sd * e4m3(Wdq) [D, H]."""
    with torch.cuda.device(x.device):
        return _glu_w8_call(x, Wgq, sg, Wuq, su, Wdq, sd, gate_act, out, workspace)()


def bind_glu_w8(x, Wgq, sg, Wuq, su, Wdq, sd, gate_act: str = "gelu_tanh", out=None,
                workspace=None) -> BoundCall:
    with torch.cuda.device(x.device):
        return _glu_w8_call(x, Wgq, sg, Wuq, su, Wdq, sd, gate_act, out, workspace)
