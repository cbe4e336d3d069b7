"""Thin ctypes binding of libgmm_mi355x.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers and torch's current HIP stream to the C-ABI, and returns
tensors the library wrote. All computation happens in the HIP kernels; there
is no CPU path. The library must have been built (``build.py``); importing
this module on a machine without it raises immediately.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgmm_mi355x.so")

GMM_F32, GMM_F16, GMM_BF16 = 0, 1, 2
REGIME_AUTO, REGIME_SINGLE, REGIME_TWOPASS, REGIME_SMALLK = 0, 1, 2, 3
STATS_FP32, STATS_SPLIT_BF16, STATS_AUTO = 0, 1, 2  # STATS_AUTO is the default

EXPORTS = (
    "gmm_version", "gmm_error_string", "gmm_workspace_bytes", "gmm_estep_stats",
    "gmm_estep_stats_regime", "gmm_estep_resp", "gmm_mstep", "gmm_em_iterate", "gmm_assign_top2",
    "gmm_set_timing_events", "gmm_set_stats_precision", "gmm_estep_stats_chunked", "gmm_workspace_bytes_chunked",
    "gmm_border_lists", "gmm_border_lists_workspace_bytes",
    "gmm_kmeans_assign", "gmm_kmeans_update", "gmm_kmeans_iterate", "gmm_kmeans_workspace_bytes",
    "gmm_plan_info", "gmm_estep_stats_static",
    "gmm_peak_mfma", "gmm_peak_mfma_flops", "gmm_peak_hbm_read", "gmm_peak_coissue",
)
PEAK_FP32, PEAK_FP64 = 0, 1


class GmmError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({error_string(code)})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with soft_clustering_gmm_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.gmm_version.restype = ctypes.c_int
    L.gmm_version.argtypes = []
    L.gmm_error_string.restype = ctypes.c_char_p
    L.gmm_error_string.argtypes = [ctypes.c_int]
    L.gmm_workspace_bytes.restype = SZ
    L.gmm_workspace_bytes.argtypes = [I64, I32, I32]
    L.gmm_estep_stats.restype = ctypes.c_int
    L.gmm_estep_stats.argtypes = [P, I32, I64, I32, P, P, P, I32, P, P, P, P, P, P, SZ, P]
    L.gmm_estep_stats_regime.restype = ctypes.c_int
    L.gmm_estep_stats_regime.argtypes = [P, I32, I64, I32, P, P, P, I32, P, P, P, P, P, P, SZ, I32, P]
    L.gmm_estep_resp.restype = ctypes.c_int
    L.gmm_estep_resp.argtypes = [P, I32, I64, I32, P, P, P, I32, P, P, P, SZ, I32, P]
    L.gmm_mstep.restype = ctypes.c_int
    L.gmm_mstep.argtypes = [P, P, P, I64, I32, I32, F32, P, P, P, P]
    L.gmm_em_iterate.restype = ctypes.c_int
    L.gmm_em_iterate.argtypes = [P, I32, I64, I32, I32, I32, F32, P, P, P, P, P, SZ, P]
    L.gmm_assign_top2.restype = ctypes.c_int
    L.gmm_assign_top2.argtypes = [P, I32, I64, I32, P, P, P, I32, P, P, P, SZ, P]
    L.gmm_set_timing_events.restype = ctypes.c_int
    L.gmm_set_timing_events.argtypes = [P, P]
    L.gmm_set_stats_precision.restype = ctypes.c_int
    L.gmm_set_stats_precision.argtypes = [ctypes.c_int32]
    L.gmm_estep_stats_chunked.restype = ctypes.c_int
    L.gmm_estep_stats_chunked.argtypes = [P, I32, I64, I32, P, P, P, I32, P, P, P, P, P, I64, P, SZ, P]
    L.gmm_workspace_bytes_chunked.restype = SZ
    L.gmm_workspace_bytes_chunked.argtypes = [I64, I32, I32, I64, I32]
    L.gmm_border_lists.restype = ctypes.c_int
    L.gmm_border_lists.argtypes = [P, P, I64, I32, F32, P, P, I64, P, SZ, P]
    L.gmm_border_lists_workspace_bytes.restype = SZ
    L.gmm_border_lists_workspace_bytes.argtypes = [I64, I32]
    L.gmm_kmeans_assign.restype = ctypes.c_int
    L.gmm_kmeans_assign.argtypes = [P, I32, I64, I32, P, I32, P, P, P, P, SZ, P]
    L.gmm_kmeans_update.restype = ctypes.c_int
    L.gmm_kmeans_update.argtypes = [P, I32, I64, I32, P, I32, P, P, P, SZ, P]
    L.gmm_kmeans_iterate.restype = ctypes.c_int
    L.gmm_kmeans_iterate.argtypes = [P, I32, I64, I32, I32, I32, P, P, P, SZ, P]
    L.gmm_kmeans_workspace_bytes.restype = SZ
    L.gmm_kmeans_workspace_bytes.argtypes = [I64, I32, I32]
    L.gmm_plan_info.restype = ctypes.c_int
    L.gmm_plan_info.argtypes = [I64, I32, I32, I32, P]
    L.gmm_peak_mfma.restype = ctypes.c_int
    L.gmm_peak_mfma.argtypes = [I32, I64, I32, P, P]
    L.gmm_peak_mfma_flops.restype = ctypes.c_double
    L.gmm_peak_mfma_flops.argtypes = [I32, I64, I32]
    L.gmm_peak_hbm_read.restype = ctypes.c_int
    L.gmm_peak_hbm_read.argtypes = [P, SZ, I32, P, P]
    L.gmm_peak_coissue.restype = ctypes.c_int
    L.gmm_peak_coissue.argtypes = [I32, I64, I32, P, P]
    L.gmm_estep_stats_static.restype = ctypes.c_int
    L.gmm_estep_stats_static.argtypes = [P, I32, I64, I32, P, P, P, I32, P, P, P, P, P, P]
    return L


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def error_string(code: int) -> str:
    return lib().gmm_error_string(code).decode()


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise GmmError(fn, code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _xtype(X: torch.Tensor) -> int:
    if X.dtype == torch.float32:
        return GMM_F32
    if X.dtype == torch.float16:
        return GMM_F16
    if X.dtype == torch.bfloat16:
        return GMM_BF16
    raise ValueError(f"X must be float32, float16 or bfloat16, got {X.dtype}")


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _params(X, mu, var, logw):
    if X.dim() != 2:
        raise ValueError("X must be N x d")
    N, d = X.shape
    K = mu.shape[0]
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("X must be on the GPU")
    _xtype(X)
    if not X.is_contiguous():
        raise ValueError("X must be contiguous")
    _need(mu, "mu", torch.float32, (K, d), dev)
    _need(var, "var", torch.float32, (K, d), dev)
    _need(logw, "logw", torch.float32, (K,), dev)
    return N, d, K, dev


def plan_info(N: int, d: int, K: int, regime: int = REGIME_AUTO) -> dict:
    """The launch shape gmm_estep_stats_regime takes for (N, d, K, regime) (host only)."""
    buf = (ctypes.c_int64 * 7)()
    _check("gmm_plan_info", lib().gmm_plan_info(N, d, K, regime, buf))
    keys = ("regime", "waves", "kslabs", "rows_per_chunk", "chunks", "tiles", "scratch_bytes")
    return dict(zip(keys, (int(v) for v in buf)))


def workspace_bytes(N: int, d: int, K: int) -> int:
    return int(lib().gmm_workspace_bytes(N, d, K))


def workspace(N: int, d: int, K: int, device) -> torch.Tensor:
    """A device workspace large enough for every entry point at (N, d, K)."""
    nb = workspace_bytes(N, d, K)
    if nb == 0:
        raise ValueError(f"unsupported shape N={N} d={d} K={K}")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _ws(ws, N, d, K, dev):
    if ws is None:
        ws = workspace(N, d, K, dev)
    return ws


def estep_stats(X, mu, var, logw, *, regime: int = REGIME_AUTO, want_point_loglik: bool = False, ws=None):
    """Fused E-step: returns (Nk[K], Sx[K,d], Sxx[K,d], L (0-d float64), l_n[N] or None)."""
    N, d, K, dev = _params(X, mu, var, logw)
    Nk = torch.empty(K, dtype=torch.float32, device=dev)
    Sx = torch.empty(K, d, dtype=torch.float32, device=dev)
    Sxx = torch.empty(K, d, dtype=torch.float32, device=dev)
    L = torch.empty((), dtype=torch.float64, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev) if want_point_loglik else None
    ws = _ws(ws, N, d, K, dev)
    _check("gmm_estep_stats_regime", lib().gmm_estep_stats_regime(
        _ptr(X), _xtype(X), N, d, _ptr(mu), _ptr(var), _ptr(logw), K, _ptr(Nk), _ptr(Sx), _ptr(Sxx),
        _ptr(L), _ptr(lp), _ptr(ws), ws.numel(), regime, _stream(dev)))
    return Nk, Sx, Sxx, L, lp


def estep_stats_static(X, mu, var, logw, *, want_point_loglik: bool = False):
    """Allocation-free fused E-step (the library's static per-GPU scratch, no
    workspace): returns the estep_stats outputs. Calls on one GPU must not overlap."""
    N, d, K, dev = _params(X, mu, var, logw)
    Nk = torch.empty(K, dtype=torch.float32, device=dev)
    Sx = torch.empty(K, d, dtype=torch.float32, device=dev)
    Sxx = torch.empty(K, d, dtype=torch.float32, device=dev)
    L = torch.empty((), dtype=torch.float64, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev) if want_point_loglik else None
    _check("gmm_estep_stats_static", lib().gmm_estep_stats_static(
        _ptr(X), _xtype(X), N, d, _ptr(mu), _ptr(var), _ptr(logw), K, _ptr(Nk), _ptr(Sx), _ptr(Sxx),
        _ptr(L), _ptr(lp), _stream(dev)))
    return Nk, Sx, Sxx, L, lp


def workspace_chunked(N: int, d: int, K: int, chunk_rows: int, x_dtype: int, device) -> torch.Tensor:
    """A device workspace for estep_stats_chunked."""
    nb = int(lib().gmm_workspace_bytes_chunked(N, d, K, chunk_rows, x_dtype))
    if nb == 0:
        raise ValueError(f"unsupported shape N={N} d={d} K={K} chunk_rows={chunk_rows}")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def estep_stats_chunked(X_host, mu, var, logw, chunk_rows: int, *, want_point_loglik: bool = False, ws=None):
    """E-step over X in host memory (a CPU tensor, ideally pinned), streamed to the
    device chunk_rows rows at a time; returns the estep_stats outputs (on mu's device)."""
    if X_host.device.type != "cpu" or X_host.dim() != 2 or not X_host.is_contiguous():
        raise ValueError("X_host must be a contiguous 2-d CPU tensor")
    N, d = X_host.shape
    K = mu.shape[0]
    dev = mu.device
    xt = _xtype(X_host)
    _need(mu, "mu", torch.float32, (K, d), dev)
    _need(var, "var", torch.float32, (K, d), dev)
    _need(logw, "logw", torch.float32, (K,), dev)
    Nk = torch.empty(K, dtype=torch.float32, device=dev)
    Sx = torch.empty(K, d, dtype=torch.float32, device=dev)
    Sxx = torch.empty(K, d, dtype=torch.float32, device=dev)
    L = torch.empty((), dtype=torch.float64, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev) if want_point_loglik else None
    if ws is None:
        ws = workspace_chunked(N, d, K, chunk_rows, xt, dev)
    _check("gmm_estep_stats_chunked", lib().gmm_estep_stats_chunked(
        _ptr(X_host), xt, N, d, _ptr(mu), _ptr(var), _ptr(logw), K, _ptr(Nk), _ptr(Sx), _ptr(Sxx), _ptr(L),
        _ptr(lp), chunk_rows, _ptr(ws), ws.numel(), _stream(dev)))
    return Nk, Sx, Sxx, L, lp


def estep_resp(X, mu, var, logw, *, regime: int = REGIME_AUTO, ws=None):
    """Testing aid: the responsibilities R[N,K] and l_n[N] from the same kernels."""
    N, d, K, dev = _params(X, mu, var, logw)
    R = torch.empty(N, K, dtype=torch.float32, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev)
    ws = _ws(ws, N, d, K, dev)
    _check("gmm_estep_resp", lib().gmm_estep_resp(
        _ptr(X), _xtype(X), N, d, _ptr(mu), _ptr(var), _ptr(logw), K, _ptr(R), _ptr(lp), _ptr(ws),
        ws.numel(), regime, _stream(dev)))
    return R, lp


def mstep(Nk, Sx, Sxx, N: int, var_floor: float, mu, var, logw):
    """In-place M-step on (mu, var, logw) from the statistics."""
    K, d = mu.shape
    dev = mu.device
    _need(Nk, "Nk", torch.float32, (K,), dev)
    _need(Sx, "Sx", torch.float32, (K, d), dev)
    _need(Sxx, "Sxx", torch.float32, (K, d), dev)
    _need(var, "var", torch.float32, (K, d), dev)
    _need(logw, "logw", torch.float32, (K,), dev)
    _check("gmm_mstep", lib().gmm_mstep(_ptr(Nk), _ptr(Sx), _ptr(Sxx), N, d, K, float(var_floor),
                                        _ptr(mu), _ptr(var), _ptr(logw), _stream(dev)))


def em_iterate(X, mu, var, logw, iters: int, var_floor: float, *, ws=None):
    """`iters` EM iterations in place; returns the log-likelihood history (device float64)."""
    N, d, K, dev = _params(X, mu, var, logw)
    hist = torch.empty(max(iters, 1), dtype=torch.float64, device=dev)
    ws = _ws(ws, N, d, K, dev)
    _check("gmm_em_iterate", lib().gmm_em_iterate(
        _ptr(X), _xtype(X), N, d, K, iters, float(var_floor), _ptr(mu), _ptr(var), _ptr(logw),
        _ptr(hist), _ptr(ws), ws.numel(), _stream(dev)))
    return hist[:iters]


def set_timing_events(start, stop) -> None:
    """One-shot: the next E-step on this thread records these torch.cuda.Events
    (already created, e.g. by one record()) around its fused kernel(s)."""
    _check("gmm_set_timing_events", lib().gmm_set_timing_events(
        None if start is None else ctypes.c_void_p(start.cuda_event),
        None if stop is None else ctypes.c_void_p(stop.cuda_event)))


def set_stats_precision(mode: int) -> None:
    """Statistics contraction of the fused E-step kernels, process-wide:
    STATS_AUTO (default: fp32 products, exact fp16 splits in the second pass over half-precision X),
    STATS_FP32 or STATS_SPLIT_BF16 (split-bf16 products)."""
    _check("gmm_set_stats_precision", lib().gmm_set_stats_precision(int(mode)))


def assign_top2(X, mu, var, logw, *, ws=None):
    """Top-2 components per point: (idx[N,2] int32, resp[N,2] float32)."""
    N, d, K, dev = _params(X, mu, var, logw)
    idx = torch.empty(N, 2, dtype=torch.int32, device=dev)
    resp = torch.empty(N, 2, dtype=torch.float32, device=dev)
    ws = _ws(ws, N, d, K, dev)
    _check("gmm_assign_top2", lib().gmm_assign_top2(
        _ptr(X), _xtype(X), N, d, _ptr(mu), _ptr(var), _ptr(logw), K, _ptr(idx), _ptr(resp),
        _ptr(ws), ws.numel(), _stream(dev)))
    return idx, resp


def border_lists(idx, resp, K: int, threshold: float, *, ws=None, members=None):
    """Inverted lists with border vectors from a top-2 assignment (idx N x 2 int32,
    resp N x 2 float32, on the GPU): returns (offsets[K+1] int64, members int32
    of capacity 2N; the lists are members[:offsets[K]])."""
    N = idx.shape[0]
    dev = idx.device
    _need(idx, "idx", torch.int32, (N, 2), dev)
    _need(resp, "resp", torch.float32, (N, 2), dev)
    offsets = torch.empty(K + 1, dtype=torch.int64, device=dev)
    if members is None:
        members = torch.empty(max(2 * N, 1), dtype=torch.int32, device=dev)
    if ws is None:
        nb = int(lib().gmm_border_lists_workspace_bytes(N, K))
        if nb == 0:
            raise ValueError(f"unsupported N={N} K={K}")
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _check("gmm_border_lists", lib().gmm_border_lists(
        _ptr(idx), _ptr(resp), N, K, float(threshold), _ptr(offsets), _ptr(members), members.numel(),
        _ptr(ws), ws.numel(), _stream(dev)))
    return offsets, members


def kmeans_workspace(N: int, d: int, K: int, device) -> torch.Tensor:
    nb = int(lib().gmm_kmeans_workspace_bytes(N, d, K))
    if nb == 0:
        raise ValueError(f"unsupported shape N={N} d={d} K={K}")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _kmeans_args(X, C):
    if X.dim() != 2 or not X.is_contiguous() or X.device.type != "cuda":
        raise ValueError("X must be a contiguous N x d GPU tensor")
    N, d = X.shape
    K = C.shape[0]
    _need(C, "C", torch.float32, (K, d), X.device)
    return N, d, K, X.device


def kmeans_assign(X, C, *, ws=None):
    """Nearest centres: (assign[N] int32, dist2[N] float32, inertia 0-d float64)."""
    N, d, K, dev = _kmeans_args(X, C)
    assign = torch.empty(N, dtype=torch.int32, device=dev)
    dist2 = torch.empty(N, dtype=torch.float32, device=dev)
    inertia = torch.empty((), dtype=torch.float64, device=dev)
    ws = kmeans_workspace(N, d, K, dev) if ws is None else ws
    _check("gmm_kmeans_assign", lib().gmm_kmeans_assign(
        _ptr(X), _xtype(X), N, d, _ptr(C), K, _ptr(assign), _ptr(dist2), _ptr(inertia), _ptr(ws), ws.numel(),
        _stream(dev)))
    return assign, dist2, inertia


def kmeans_update(X, assign, C, *, ws=None):
    """In-place centre update from a hard assignment; returns the counts (int64 K)."""
    N, d, K, dev = _kmeans_args(X, C)
    _need(assign, "assign", torch.int32, (N,), dev)
    counts = torch.empty(K, dtype=torch.int64, device=dev)
    ws = kmeans_workspace(N, d, K, dev) if ws is None else ws
    _check("gmm_kmeans_update", lib().gmm_kmeans_update(
        _ptr(X), _xtype(X), N, d, _ptr(assign), K, _ptr(C), _ptr(counts), _ptr(ws), ws.numel(), _stream(dev)))
    return counts


def kmeans_iterate(X, C, iters: int, *, ws=None):
    """`iters` Lloyd iterations in place on C; returns the inertia history (device float64)."""
    N, d, K, dev = _kmeans_args(X, C)
    hist = torch.empty(max(iters, 1), dtype=torch.float64, device=dev)
    ws = kmeans_workspace(N, d, K, dev) if ws is None else ws
    _check("gmm_kmeans_iterate", lib().gmm_kmeans_iterate(
        _ptr(X), _xtype(X), N, d, K, iters, _ptr(C), _ptr(hist), _ptr(ws), ws.numel(), _stream(dev)))
    return hist[:iters]


def peak_mfma(precision: int, trips: int, blocks: int, out: torch.Tensor) -> float:
    """Enqueues the matrix-core issue loop on the current stream; returns the flops it executes."""
    _check("gmm_peak_mfma", lib().gmm_peak_mfma(precision, trips, blocks, _ptr(out), _stream(out.device)))
    return float(lib().gmm_peak_mfma_flops(precision, trips, blocks))


def peak_hbm_read(buf: torch.Tensor, blocks: int, out: torch.Tensor) -> int:
    """Enqueues the HBM read stream over buf on the current stream; returns the bytes it reads."""
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    _check("gmm_peak_hbm_read", lib().gmm_peak_hbm_read(_ptr(buf), nbytes, blocks, _ptr(out), _stream(buf.device)))
    return nbytes


def peak_coissue(mode: int, trips: int, blocks: int, out: torch.Tensor) -> None:
    """Enqueues the co-issue probe (0 matrix only, 1 vector only, 2 both per wave, 3 split waves)."""
    _check("gmm_peak_coissue", lib().gmm_peak_coissue(mode, trips, blocks, _ptr(out), _stream(out.device)))
