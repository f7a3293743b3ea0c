"""Python binding of libgmm_em.so (argument marshalling only).

Every step of the EM path runs in the HIP library; this module only checks
tensor shapes, dtypes and devices, allocates the workspace with PyTorch and
passes raw device pointers and the current HIP stream through the C ABI
declared in ``include/gmm_em.h``. Importing it fails loudly when the library
has not been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgmm_em.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built: run `python -m gmm_em_amd.build`")
lib = ctypes.CDLL(_LIB_PATH)

_vp, _i64, _i32, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
lib.gmm_workspace_bytes.argtypes = [_i32, _i32]
lib.gmm_workspace_bytes.restype = _sz
lib.gmm_em_step.argtypes = [_vp, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _i32, _f32, _vp, _vp, _sz, _vp]
lib.gmm_fit.argtypes = [_vp, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _i32, _f32, _i32, _f64, _vp,
                        ctypes.POINTER(_i32), _vp, _sz, _vp]
lib.gmm_loglik.argtypes = [_vp, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]
lib.gmm_assign_topm.argtypes = [_vp, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _vp,
                                _vp, _sz, _vp]
lib.gmm_kmeans_step.argtypes = [_vp, _i64, _i32, _i64, _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]
lib.gmm_kmeans_fit.argtypes = [_vp, _i64, _i32, _i64, _i32, _vp, _i32, _i32, _f64, _vp,
                               ctypes.POINTER(_i32), _vp, _sz, _vp]
lib.gmm_ivf_workspace_bytes.argtypes = [_i64, _i32, _i32]
lib.gmm_ivf_workspace_bytes.restype = _sz
lib.gmm_ivf_build.argtypes = [_vp, _vp, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]
lib.gmm_device_status.argtypes = [_vp, _vp]
lib.gmm_estep_arithmetic.argtypes = [_vp, _vp]
lib.gmm_estep_arithmetic.restype = ctypes.c_int
lib.gmm_status_string.argtypes = [ctypes.c_int]
lib.gmm_status_string.restype = ctypes.c_char_p
lib.gmm_version.restype = _i32
lib.gmm_profile_begin.argtypes = [_i32]
lib.gmm_profile_end.argtypes = [ctypes.POINTER(_f64), ctypes.POINTER(_i32), ctypes.POINTER(_f64),
                                ctypes.POINTER(_i32)]
for _f in (lib.gmm_em_step, lib.gmm_fit, lib.gmm_loglik, lib.gmm_assign_topm, lib.gmm_kmeans_step,
           lib.gmm_kmeans_fit, lib.gmm_ivf_build, lib.gmm_device_status, lib.gmm_profile_begin,
           lib.gmm_profile_end):
    _f.restype = ctypes.c_int

(GMM_OK, GMM_E_INVALID, GMM_E_DTYPE, GMM_E_WORKSPACE, GMM_E_PARAMS, GMM_E_HIP,
 GMM_E_UNSUPPORTED) = range(7)
GMM_F32, GMM_BF16 = 0, 1  # gmm_dtype


class GmmError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(f"gmm_em: {lib.gmm_status_string(code).decode()} (status {code})")


def _check(rc: int) -> None:
    if rc != GMM_OK:
        raise GmmError(rc)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(d: int, k: int) -> int:
    return int(lib.gmm_workspace_bytes(d, k))


def workspace(d: int, k: int, device="cuda") -> torch.Tensor:
    """A workspace buffer for data of dimension d with k components."""
    nb = workspace_bytes(d, k)
    if nb == 0:
        raise GmmError(GMM_E_UNSUPPORTED)
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _data(x: torch.Tensor):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit stride along columns")
    if x.dtype == torch.float32:
        dt = GMM_F32
    elif x.dtype == torch.bfloat16:
        dt = GMM_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    return dt, max(x.stride(0), x.shape[1])


def _params(x, w, mu, var):
    k, d = mu.shape
    for t, shape in ((w, (k,)), (mu, (k, d)), (var, (k, d))):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError("parameters must be contiguous float32: weights (K,), means/variances (K, D)")
        if t.device != x.device:
            raise ValueError("parameters must be on the device of x")
    if x.shape[1] != d:
        raise ValueError("x and means disagree on D")
    return k, d


def _ws(ws, d, k, device):
    return workspace(d, k, device) if ws is None else ws


def em_step(x, weights, means, variances, var_floor: float = 1e-6, ws=None, loglik=None):
    """One EM iteration in place; returns the 0-d float64 device tensor L(input params)."""
    dt, ldx = _data(x)
    k, d = _params(x, weights, means, variances)
    ws = _ws(ws, d, k, x.device)
    out = torch.empty((), dtype=torch.float64, device=x.device) if loglik is None else loglik
    _check(lib.gmm_em_step(_ptr(x), x.shape[0], d, ldx, dt, _ptr(weights), _ptr(means),
                           _ptr(variances), k, var_floor, _ptr(out), _ptr(ws), ws.numel(),
                           _stream(x.device)))
    return out


def fit(x, weights, means, variances, var_floor: float = 1e-6, max_iter: int = 10,
        tol: float = 0.0, ws=None):
    """EM iterations in place; returns (history float64 tensor of L(theta_t), iterations)."""
    dt, ldx = _data(x)
    k, d = _params(x, weights, means, variances)
    ws = _ws(ws, d, k, x.device)
    hist = torch.full((max(max_iter, 1),), float("nan"), dtype=torch.float64, device=x.device)
    done = _i32(0)
    _check(lib.gmm_fit(_ptr(x), x.shape[0], d, ldx, dt, _ptr(weights), _ptr(means), _ptr(variances),
                       k, var_floor, max_iter, tol, _ptr(hist), ctypes.byref(done), _ptr(ws),
                       ws.numel(), _stream(x.device)))
    return hist[: done.value], done.value


def loglik(x, weights, means, variances, per_row: bool = False, ws=None):
    """Total log-likelihood (0-d float64 device tensor) and optionally per-row values."""
    dt, ldx = _data(x)
    k, d = _params(x, weights, means, variances)
    ws = _ws(ws, d, k, x.device)
    total = torch.empty((), dtype=torch.float64, device=x.device)
    rows = torch.empty(x.shape[0], dtype=torch.float64, device=x.device) if per_row else None
    _check(lib.gmm_loglik(_ptr(x), x.shape[0], d, ldx, dt, _ptr(weights), _ptr(means),
                          _ptr(variances), k, _ptr(total), _ptr(rows), _ptr(ws), ws.numel(),
                          _stream(x.device)))
    return (total, rows) if per_row else total


def assign_topm(x, weights, means, variances, m: int = 2, ws=None):
    """Top-m components per row by responsibility: (idx int32 (N, m), resp float32 (N, m))."""
    dt, ldx = _data(x)
    k, d = _params(x, weights, means, variances)
    ws = _ws(ws, d, k, x.device)
    idx = torch.empty((x.shape[0], m), dtype=torch.int32, device=x.device)
    resp = torch.empty((x.shape[0], m), dtype=torch.float32, device=x.device)
    _check(lib.gmm_assign_topm(_ptr(x), x.shape[0], d, ldx, dt, _ptr(weights), _ptr(means),
                               _ptr(variances), k, m, _ptr(idx), _ptr(resp), _ptr(ws), ws.numel(),
                               _stream(x.device)))
    return idx, resp


def kmeans_step(x, centroids, ws=None, assign: bool = True):
    """One Lloyd step in place on centroids (K, D) float32.

    Returns (inertia 0-d float64 device tensor for the input centroids,
    assignment int32 (N,) or None).
    """
    dt, ldx = _data(x)
    if centroids.dtype != torch.float32 or not centroids.is_contiguous() or centroids.dim() != 2:
        raise ValueError("centroids must be a contiguous float32 (K, D) tensor")
    if centroids.device != x.device or centroids.shape[1] != x.shape[1]:
        raise ValueError("centroids must be on the device of x and match its D")
    k, d = centroids.shape
    ws = _ws(ws, d, k, x.device)
    inertia = torch.empty((), dtype=torch.float64, device=x.device)
    z = torch.empty(x.shape[0], dtype=torch.int32, device=x.device) if assign else None
    _check(lib.gmm_kmeans_step(_ptr(x), x.shape[0], d, ldx, dt, _ptr(centroids), k, _ptr(z),
                               _ptr(inertia), _ptr(ws), ws.numel(), _stream(x.device)))
    return inertia, z


def kmeans_fit(x, centroids, max_iter: int = 10, tol: float = 0.0, ws=None):
    """Lloyd steps in place; returns (inertia history float64 tensor, steps taken)."""
    dt, ldx = _data(x)
    if centroids.dtype != torch.float32 or not centroids.is_contiguous() or centroids.dim() != 2:
        raise ValueError("centroids must be a contiguous float32 (K, D) tensor")
    if centroids.device != x.device or centroids.shape[1] != x.shape[1]:
        raise ValueError("centroids must be on the device of x and match its D")
    k, d = centroids.shape
    ws = _ws(ws, d, k, x.device)
    hist = torch.full((max(max_iter, 1),), float("nan"), dtype=torch.float64, device=x.device)
    done = _i32(0)
    _check(lib.gmm_kmeans_fit(_ptr(x), x.shape[0], d, ldx, dt, _ptr(centroids), k, max_iter, tol,
                              _ptr(hist), ctypes.byref(done), _ptr(ws), ws.numel(),
                              _stream(x.device)))
    return hist[: done.value], done.value


def ivf_build(idx, resp, k: int, min_resp: float = 0.0, values: bool = True):
    """Inverted lists from top-m assignments idx (N, m) int32 / resp (N, m) float32.

    Returns (offsets int64 (k+1,), rows int32 (entries,), values float32 or
    None); list c is rows[offsets[c]:offsets[c+1]]. Synchronises once to
    size the outputs to the entries stored.
    """
    if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous() or not idx.is_cuda:
        raise ValueError("idx must be a contiguous int32 (N, m) device tensor")
    if resp is not None and (resp.dtype != torch.float32 or tuple(resp.shape) != tuple(idx.shape)
                             or not resp.is_contiguous() or resp.device != idx.device):
        raise ValueError("resp must be a contiguous float32 tensor shaped like idx")
    n, m = idx.shape
    nb = int(lib.gmm_ivf_workspace_bytes(n, m, k))
    if nb == 0:
        raise GmmError(GMM_E_UNSUPPORTED)
    dev = idx.device
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    offsets = torch.empty(k + 1, dtype=torch.int64, device=dev)
    rows = torch.empty(max(n * m, 1), dtype=torch.int32, device=dev)
    vals = torch.empty(max(n * m, 1), dtype=torch.float32, device=dev) if values else None
    _check(lib.gmm_ivf_build(_ptr(idx), _ptr(resp), n, m, k, min_resp, _ptr(offsets), _ptr(rows),
                             _ptr(vals), _ptr(ws), nb, _stream(dev)))
    total = int(offsets[k].item())
    return offsets, rows[:total], (vals[:total] if values else None)


def device_status(ws, device="cuda") -> int:
    """Synchronise and return the status of the last call that used ``ws``."""
    return int(lib.gmm_device_status(_ptr(ws), _stream(torch.device(device))))


(GMM_ESTEP_FP64, GMM_ESTEP_INT8_SLICES, GMM_ESTEP_INT8_SLICES_BOTH, GMM_ESTEP_INT8_SLICES_MSTEP,
 GMM_ESTEP_BF16_SPLIT) = 0, 1, 2, 3, 4


def estep_arithmetic(ws, device="cuda") -> int:
    """Synchronise; the gmm_estep_kind of the last EM step / log-likelihood /
    k-means / top-m assignment call on ``ws``: GMM_ESTEP_FP64, GMM_ESTEP_INT8_SLICES (normaliser pass on exact
    int8 slices), GMM_ESTEP_INT8_SLICES_BOTH (both passes) or
    GMM_ESTEP_INT8_SLICES_MSTEP (both passes, and the M-step too) or
    GMM_ESTEP_BF16_SPLIT (bf16 data: both passes on split bf16)."""
    return int(lib.gmm_estep_arithmetic(_ptr(ws), _stream(torch.device(device))))


def profile_begin(max_launches: int = 4096) -> None:
    """Record HIP events around every pass-1/pass-2 launch until profile_end()."""
    _check(lib.gmm_profile_begin(max_launches))


def profile_end():
    """Returns {"pass1": (total_ms, launches), "pass2": (total_ms, launches)}."""
    a, b, na, nb = _f64(0), _f64(0), _i32(0), _i32(0)
    _check(lib.gmm_profile_end(ctypes.byref(a), ctypes.byref(na), ctypes.byref(b), ctypes.byref(nb)))
    return {"pass1": (a.value, na.value), "pass2": (b.value, nb.value)}
