"""Exact Lloyd k-means on MI355X (gfx950): Python binding of libflashkm.so.

The functions below only marshal torch tensors into the C ABI declared in
``include/flashkm.h`` (same names without the ``kmeans_`` prefix): every step
of the computation runs in the library's HIP kernels, on the current torch
stream.  PyTorch provides device memory and streams, nothing else.  There is
no CPU fallback: importing raises if the library is missing, and every call
raises ``KMeansError`` on a non-zero status.

Shapes: X is [N, D] or [B, N, D] (fp32 / fp16 / bf16, CUDA, contiguous);
centroids are [K, D] or [B, K, D] fp32.
"""

from __future__ import annotations

import ctypes
import functools
import os

import torch

__all__ = ["KMeansError", "lib_path", "workspace_bytes", "assign", "assign_top2", "assign_soft", "gauss_sum", "seed", "update",
           "fit", "fit_streamed", "tune", "tune_save", "tune_load", "assign_configs", "assign_noalloc",
           "stream_timeline", "DTYPES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libflashkm.so"

KM_OK, KM_EINVAL, KM_EUNSUPPORTED, KM_EWORKSPACE, KM_EHIP, KM_ENOMEM = range(6)
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class KMeansError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"flashkm status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _load(path=None):
    path = path or lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python exact_means_clustering_amd/build.py` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kmeans_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.kmeans_workspace_bytes.restype = sz
    lib.kmeans_assign.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P, sz, P]
    lib.kmeans_assign.restype = ctypes.c_int
    lib.kmeans_assign_noalloc.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P]
    lib.kmeans_assign_noalloc.restype = ctypes.c_int
    lib.kmeans_update.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P, sz, P]
    lib.kmeans_update.restype = ctypes.c_int
    lib.kmeans_fit.argtypes = [P, i32, i64, i32, i32, P, i32, i32, P, P, P, P, P, sz, P]
    lib.kmeans_fit.restype = ctypes.c_int
    lib.kmeans_fit_streamed.argtypes = [P, i32, i64, i32, P, i32, i32, sz, P, P, P, P, P]
    lib.kmeans_fit_streamed.restype = ctypes.c_int
    lib.kmeans_assign_top2.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, sz, P]
    lib.kmeans_assign_top2.restype = ctypes.c_int
    lib.kmeans_assign_soft.argtypes = [P, i32, i64, i32, i32, P, i32, P, ctypes.c_float, P, P, P, P, sz, P]
    lib.kmeans_assign_soft.restype = ctypes.c_int
    lib.kmeans_gauss_sum.argtypes = [P, i32, i64, i32, i32, P, i32, P, ctypes.c_float, P, P, P, sz, P]
    lib.kmeans_gauss_sum.restype = ctypes.c_int
    lib.kmeans_seed.argtypes = [P, i32, i64, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.kmeans_seed.restype = ctypes.c_int
    lib.kmeans_tune.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, sz, P, P, P, P]
    lib.kmeans_tune.restype = ctypes.c_int
    lib.kmeans_tune_save.argtypes = [ctypes.c_char_p]
    lib.kmeans_tune_save.restype = ctypes.c_int
    lib.kmeans_assign_configs.argtypes = [i32, i32, P, P, i32, P]
    lib.kmeans_stream_timeline.argtypes = [P, i32, P]
    lib.kmeans_stream_timeline.restype = ctypes.c_int
    lib.kmeans_assign_configs.restype = ctypes.c_int
    lib.kmeans_tune_load.argtypes = [ctypes.c_char_p]
    lib.kmeans_tune_load.restype = ctypes.c_int
    lib.kmeans_last_error.argtypes = []
    lib.kmeans_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _check(rc: int):
    if rc != KM_OK:
        raise KMeansError(rc, _lib.kmeans_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _shape3(X):
    if X.dim() == 2:
        return 1, X.shape[0], X.shape[1]
    if X.dim() == 3:
        return X.shape
    raise ValueError("X must be [N, D] or [B, N, D]")


def _dtype(X):
    try:
        return DTYPES[X.dtype]
    except KeyError:
        raise KMeansError(KM_EUNSUPPORTED, f"unsupported dtype {X.dtype}") from None


def _need(t, name, dtype=None, like=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise KMeansError(KM_EINVAL, f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise KMeansError(KM_EINVAL, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KMeansError(KM_EINVAL, f"{name} must be {dtype}")
    if like is not None and t.device != like.device:
        raise KMeansError(KM_EINVAL, f"{name} must be on {like.device} (it is on {t.device})")


def _on_tensor_device(fn):
    """Run fn with its first CUDA tensor argument's device current, so the
    default stream and the library's device queries belong to that device."""
    @functools.wraps(fn)
    def run(*args, **kwargs):
        for a in args:
            if isinstance(a, torch.Tensor) and a.is_cuda:
                with torch.cuda.device(a.device):
                    return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return run


def _rows(C, name, B, D):
    """K of a centroid-like tensor [K, D] (B = 1) or [B, K, D] that goes with X."""
    ok = C.shape[-1] == D and (C.dim() == 3 and C.shape[0] == B or C.dim() == 2 and B == 1)
    if not ok:
        raise KMeansError(KM_EINVAL, f"{name} must be [K, {D}] or [{B}, K, {D}] (got {tuple(C.shape)})")
    return C.shape[-2]


def _count(t, name, n):
    if t.numel() != n:
        raise KMeansError(KM_EINVAL, f"{name} must have {n} elements (got {t.numel()})")


def workspace_bytes(N: int, D: int, K: int, B: int = 1, dtype=torch.bfloat16) -> int:
    dt = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.kmeans_workspace_bytes(N, D, K, B, dt))


def _workspace(N, D, K, B, dt, device, ws):
    """A caller workspace (any dtype, contiguous, on X's device) or a new one;
    returns (tensor, its size in bytes)."""
    need = int(_lib.kmeans_workspace_bytes(N, D, K, B, dt))
    if need == 0:
        _check(_lib.kmeans_workspace_bytes(N, D, K, B, dt) or KM_EINVAL)
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device or not ws.is_contiguous():
            raise KMeansError(KM_EINVAL, f"ws must be a contiguous tensor on {device}")
        if ws.numel() * ws.element_size() >= need:
            return ws, ws.numel() * ws.element_size()
    return torch.empty(need, dtype=torch.uint8, device=device), need


@_on_tensor_device
def assign(X, C, *, want_min_d2: bool = False, ws=None, stream=None, labels=None):
    """Assignment stage: returns (labels int32, min_d2 fp32 or None, inertia fp64 [B])."""
    _need(X, "X")
    _need(C, "C", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C, "C", B, D)
    dt = _dtype(X)
    lab_shape = X.shape[:-1]
    if labels is None:
        labels = torch.empty(lab_shape, dtype=torch.int32, device=X.device)
    else:
        _need(labels, "labels", torch.int32, like=X)
        _count(labels, "labels", B * N)
    md = torch.empty(lab_shape, dtype=torch.float32, device=X.device) if want_min_d2 else None
    inertia = torch.empty(B, dtype=torch.float64, device=X.device)
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_assign(_ptr(X), dt, N, D, B, _ptr(C), K, _ptr(labels), _ptr(md), _ptr(inertia),
                              _ptr(ws), ws_bytes, _stream(stream)))
    return labels, md, inertia


@_on_tensor_device
def assign_noalloc(X, C, *, labels, inertia, min_d2=None, stream=None):
    """Assignment stage into caller tensors with no workspace and no allocation (the library's static
    scratch; calls that overlap on one GPU race): labels int32 [.., N], inertia fp64 [B], min_d2 fp32 [.., N]
    or None.  Returns (labels, min_d2, inertia)."""
    _need(X, "X")
    _need(C, "C", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C, "C", B, D)
    dt = _dtype(X)
    _need(labels, "labels", torch.int32, like=X)
    _count(labels, "labels", B * N)
    _need(inertia, "inertia", torch.float64, like=X)
    _count(inertia, "inertia", B)
    if min_d2 is not None:
        _need(min_d2, "min_d2", torch.float32, like=X)
        _count(min_d2, "min_d2", B * N)
    _check(_lib.kmeans_assign_noalloc(_ptr(X), dt, N, D, B, _ptr(C), K, _ptr(labels), _ptr(min_d2), _ptr(inertia),
                                      _stream(stream)))
    return labels, min_d2, inertia


@_on_tensor_device
def assign_top2(X, C, *, ws=None, stream=None):
    """Two nearest centroids of every point: returns (labels [.., N, 2] int32, distances [.., N, 2] fp32)."""
    _need(X, "X")
    _need(C, "C", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C, "C", B, D)
    dt = _dtype(X)
    labels2 = torch.empty((*X.shape[:-1], 2), dtype=torch.int32, device=X.device)
    d2 = torch.empty((*X.shape[:-1], 2), dtype=torch.float32, device=X.device)
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_assign_top2(_ptr(X), dt, N, D, B, _ptr(C), K, _ptr(labels2), _ptr(d2), _ptr(ws), ws_bytes,
                                   _stream(stream)))
    return labels2, d2


@_on_tensor_device
def assign_soft(X, C, sigma2: float, *, log_w=None, ws=None, stream=None):
    """Gaussian-mixture soft assignment (shared variance sigma2, log-weights log_w [.., K] or None): returns
    (most responsible component int32, log density fp32, its per-instance sum fp64 [B])."""
    _need(X, "X")
    _need(C, "C", torch.float32, like=X)
    if log_w is not None:
        _need(log_w, "log_w", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C, "C", B, D)
    if log_w is not None:
        _count(log_w, "log_w", B * K)
    dt = _dtype(X)
    labels = torch.empty(X.shape[:-1], dtype=torch.int32, device=X.device)
    logp = torch.empty(X.shape[:-1], dtype=torch.float32, device=X.device)
    total = torch.empty(B, dtype=torch.float64, device=X.device)
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_assign_soft(_ptr(X), dt, N, D, B, _ptr(C), K, _ptr(log_w), float(sigma2), _ptr(labels),
                                   _ptr(logp), _ptr(total), _ptr(ws), ws_bytes, _stream(stream)))
    return labels, logp, total


@_on_tensor_device
def gauss_sum(X, Y, w, sigma2: float, *, ws=None, stream=None):
    """Gauss kernel sums G[.., i] = sum_k w[.., k] exp(-||x_i - y_k||^2 / (2 sigma2)): returns (G fp32, sum fp64 [B])."""
    _need(X, "X")
    _need(Y, "Y", torch.float32, like=X)
    _need(w, "w", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(Y, "Y", B, D)
    _count(w, "w", B * K)
    dt = _dtype(X)
    G = torch.empty(X.shape[:-1], dtype=torch.float32, device=X.device)
    total = torch.empty(B, dtype=torch.float64, device=X.device)
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_gauss_sum(_ptr(X), dt, N, D, B, _ptr(Y), K, _ptr(w), float(sigma2), _ptr(G), _ptr(total),
                                 _ptr(ws), ws_bytes, _stream(stream)))
    return G, total


@_on_tensor_device
def seed(X, u, *, method: str = "kmeans++", want_d2: bool = False, ws=None, stream=None):
    """Initial centroids from the caller's uniforms u [.., K] (fp64, CUDA, in [0, 1)): method "random" (rows
    floor(u N)) or "kmeans++" (D^2 sampling).  Returns (row indices int32 [.., K], centroids fp32 [.., K, D],
    squared distance of every row to its nearest pick fp32 [.., N] or None)."""
    _need(X, "X")
    _need(u, "u", torch.float64, like=X)
    B, N, D = _shape3(X)
    K = u.shape[-1]
    if u.numel() != B * K:
        raise KMeansError(KM_EINVAL, "u must be [K] or [B, K]")
    dt = _dtype(X)
    m = {"random": 0, "kmeans++": 1}.get(method)
    if m is None:
        raise KMeansError(KM_EINVAL, f"unknown seeding method {method!r}")
    idx = torch.empty(u.shape, dtype=torch.int32, device=X.device)
    C = torch.empty((*u.shape, D), dtype=torch.float32, device=X.device)
    d2 = torch.empty(X.shape[:-1], dtype=torch.float32, device=X.device) if want_d2 else None
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_seed(_ptr(X), dt, N, D, B, K, m, _ptr(u), _ptr(idx), _ptr(C), _ptr(d2), _ptr(ws), ws_bytes,
                            _stream(stream)))
    return idx, C, d2


@_on_tensor_device
def update(X, labels, C_prev, *, C_new=None, ws=None, stream=None):
    """Centroid update stage: returns (C_new fp32, counts int32)."""
    _need(X, "X")
    _need(labels, "labels", torch.int32, like=X)
    _need(C_prev, "C_prev", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C_prev, "C_prev", B, D)
    _count(labels, "labels", B * N)
    dt = _dtype(X)
    if C_new is None:
        C_new = torch.empty_like(C_prev)
    else:
        _need(C_new, "C_new", torch.float32, like=X)
        _count(C_new, "C_new", B * K * D)
    counts = torch.empty(C_prev.shape[:-1], dtype=torch.int32, device=X.device)
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_update(_ptr(X), dt, N, D, B, _ptr(labels), K, _ptr(C_prev), _ptr(C_new), _ptr(counts),
                              _ptr(ws), ws_bytes, _stream(stream)))
    return C_new, counts


@_on_tensor_device
def fit(X, C0, iters: int, *, history: bool = False, ws=None, stream=None, out=None):
    """Exact Lloyd iteration: returns (labels, C, inertia [B] fp64, history [iters, B] or None).

    ``out`` = (labels, C, inertia, history-or-None) reuses caller tensors for the results: calls with the same
    buffers replay the library's captured graph of the fit instead of capturing a new one."""
    _need(X, "X")
    _need(C0, "C0", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C0, "C0", B, D)
    dt = _dtype(X)
    if out is not None:
        labels, C, inertia, hist = out
        _need(labels, "labels", torch.int32, like=X)
        _need(C, "C", torch.float32, like=X)
        _need(inertia, "inertia", torch.float64, like=X)
        if labels.numel() != B * N or C.numel() != B * K * D or inertia.numel() != B:
            raise KMeansError(KM_EINVAL, "out tensors do not match the problem's shapes")
        if history:
            if hist is None or hist.numel() < max(1, int(iters)) * B:
                raise KMeansError(KM_EINVAL, "history requested but out[3] is missing or too small")
            _need(hist, "history", torch.float64, like=X)
        else:
            hist = None
    else:
        labels = torch.empty(X.shape[:-1], dtype=torch.int32, device=X.device)
        C = torch.empty_like(C0)
        inertia = torch.empty(B, dtype=torch.float64, device=X.device)
        hist = torch.empty((max(1, int(iters)), B), dtype=torch.float64, device=X.device) if history else None
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    _check(_lib.kmeans_fit(_ptr(X), dt, N, D, B, _ptr(C0), K, int(iters), _ptr(labels), _ptr(C), _ptr(inertia),
                           _ptr(hist), _ptr(ws), ws_bytes, _stream(stream)))
    return labels, C, inertia, hist


@_on_tensor_device
def tune(X, C, *, labels=None, ws=None, stream=None):
    """Time every compiled assignment configuration on this shape and record the
    fastest in the library's tuning table.  Returns (pb, waves, ms per launch)."""
    _need(X, "X")
    _need(C, "C", torch.float32, like=X)
    B, N, D = _shape3(X)
    K = _rows(C, "C", B, D)
    dt = _dtype(X)
    if labels is None:
        labels = torch.empty(X.shape[:-1], dtype=torch.int32, device=X.device)
    else:
        _need(labels, "labels", torch.int32, like=X)
        _count(labels, "labels", B * N)
    ws, ws_bytes = _workspace(N, D, K, B, dt, X.device, ws)
    pb, waves, ms = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_float(0.0)
    _check(_lib.kmeans_tune(_ptr(X), dt, N, D, B, _ptr(C), K, _ptr(labels), _ptr(ws), ws_bytes, _stream(stream),
                            ctypes.byref(pb), ctypes.byref(waves), ctypes.byref(ms)))
    return pb.value, waves.value, ms.value


def tune_save(path: str):
    """Write the tuning table as text ("dtype D N B K pb waves" per line)."""
    _check(_lib.kmeans_tune_save(os.fsencode(path)))


def assign_configs(dtype, D: int) -> list:
    """The (pb, waves) assignment configurations compiled for rows of D elements of dtype."""
    dt = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    pb, waves, n = (ctypes.c_int32 * 8)(), (ctypes.c_int32 * 8)(), ctypes.c_int32(0)
    _check(_lib.kmeans_assign_configs(dt, int(D), pb, waves, 8, ctypes.byref(n)))
    if n.value > 8:
        raise KMeansError(KM_EINVAL, f"{n.value} configurations; the binding reads at most 8")
    return [(pb[i], waves[i]) for i in range(n.value)]


def stream_timeline():
    """Per-chunk timeline of the last fit_streamed on this thread: a list of rows (iteration, chunk, copy-in start,
    copy-in end, compute start, compute end, labels-out start, labels-out end), times in ms from the fit's start."""
    n = ctypes.c_int32(0)
    _check(_lib.kmeans_stream_timeline(None, 0, ctypes.byref(n)))
    buf = (ctypes.c_double * (8 * max(1, n.value)))()
    _check(_lib.kmeans_stream_timeline(buf, n.value, ctypes.byref(n)))
    return [tuple(buf[8 * i + j] for j in range(8)) for i in range(n.value)]


def tune_load(path: str):
    """Add the entries of a tuning-table file (all or nothing)."""
    _check(_lib.kmeans_tune_load(os.fsencode(path)))


@_on_tensor_device
def fit_streamed(X_host, C0, iters: int, device_x_budget: int, *, history: bool = False, stream=None):
    """Out-of-core Lloyd iteration over a pinned host tensor X_host [N, D].

    Returns (labels int32 CPU, C fp32 CUDA, inertia float, history list or None)."""
    if not isinstance(X_host, torch.Tensor) or X_host.is_cuda or not X_host.is_pinned():
        raise KMeansError(KM_EINVAL, "X_host must be a pinned CPU tensor")
    if X_host.dim() != 2 or not X_host.is_contiguous():
        raise KMeansError(KM_EINVAL, "X_host must be a contiguous [N, D] tensor")
    _need(C0, "C0", torch.float32)
    N, D = X_host.shape
    K = _rows(C0, "C0", 1, D)
    dt = _dtype(X_host)
    labels = torch.empty(N, dtype=torch.int32, pin_memory=True)
    C = torch.empty_like(C0)
    inertia = ctypes.c_double(0.0)
    hist = (ctypes.c_double * max(1, int(iters)))() if history else None
    _check(_lib.kmeans_fit_streamed(_ptr(X_host), dt, N, D, _ptr(C0), K, int(iters), int(device_x_budget),
                                    _ptr(labels), _ptr(C), ctypes.byref(inertia),
                                    hist if hist is not None else None, _stream(stream)))
    return labels, C, inertia.value, (list(hist) if hist is not None else None)
