"""fp64 CPU oracle for one EM iteration of a diagonal-covariance GMM.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The HIP library and
its Python binding never import it, and it imports nothing from them.

Two independent implementations of the same definition live here:

* ``em_step`` / ``loglik`` / ``topm`` / ``logdensity`` call the plain C code in
  ``gmm_oracle.c`` (fp64, direct (x - mu)^2 form, fixed-block ordered sums);
* ``brute_em_step`` materialises the whole N x K responsibility matrix in
  numpy fp64 and uses the two-pass variance; it is for tiny inputs only and
  serves as a cross-check of the streaming C code.

``kmeans_step`` (C) is one Lloyd step, the hard-assignment quantizer the
pages compare the GMM with (same source, section 3).

``ivf_lists`` (numpy) builds the inverted lists of an IVF coarse quantizer
from soft top-m assignments: border vectors stored in several lists, as the
Flash-GMM abstract describes for the GMM-based quantizer.

The EM definition followed is the textbook diagonal-covariance one that the
Flash-GMM pages tile ("Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
Clustering", section 1, responsibility matrix; section 3, EM with per-tile
statistics accumulated globally). The pages print no formulas; the steps are
written out at the top of ``gmm_oracle.c``. Readings where the pages are
silent: diagonal covariance; the reported log-likelihood is the total over
rows for the step's input parameters; the variance floor is a clamp applied
after the M-step; a component with zero responsibility mass keeps its mean and
variance and gets weight 0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gmm_oracle.c")
LIB_FAST = os.path.join(HERE, "libgmm_oracle.so")  # x86-64-v3 (AVX2)
LIB_BASE = os.path.join(HERE, "libgmm_oracle_base.so")  # baseline x86-64

_FLAGS = ["-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11"]


def build() -> None:
    """Compile the oracle library (both the AVX2 and the baseline variant)."""
    for out, arch in ((LIB_FAST, "-march=x86-64-v3"), (LIB_BASE, "-march=x86-64")):
        tmp = out + ".tmp"
        subprocess.run(["gcc", *_FLAGS, arch, SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)


def _cpu_has_avx2() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("flags"):
                    flags = line.split()
                    return "avx2" in flags and "fma" in flags
    except OSError:
        pass
    return False


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = LIB_FAST if _cpu_has_avx2() else LIB_BASE
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    fp = ctypes.POINTER(ctypes.c_float)
    ip = ctypes.POINTER(ctypes.c_int32)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_loglik.argtypes = [fp, i64, i32, i32, dp, dp, dp, dp, dp]
    lib.oracle_logdensity.argtypes = [fp, i64, i32, i32, dp, dp, dp, dp]
    lib.oracle_em_step.argtypes = [fp, i64, i32, i32, dp, dp, dp, dbl, dp, dp, dp, dp, dp]
    lib.oracle_topm.argtypes = [fp, i64, i32, i32, dp, dp, dp, i32, ip, dp, dp]
    lib.oracle_kmeans_step.argtypes = [fp, i64, i32, i32, dp, dp, ip, dp, dp]
    for f in (lib.oracle_loglik, lib.oracle_logdensity, lib.oracle_em_step, lib.oracle_topm,
              lib.oracle_kmeans_step):
        f.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


_ERRORS = {1: "invalid sizes", 2: "invalid parameters", 3: "out of memory"}


def _check(rc: int) -> None:
    if rc:
        raise OracleError(_ERRORS.get(rc, f"error {rc}"))


def _x32(x: np.ndarray) -> np.ndarray:
    """Rows as contiguous fp32; bf16 bit patterns (uint16) are widened exactly."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if x.dtype != np.float32:
        raise TypeError("oracle rows must be float32 or bf16 bit patterns")
    return np.ascontiguousarray(x)


def _p64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def em_step(x, w, mu, var, var_floor: float = 1e-6):
    """One EM iteration. Returns (w', mu', var', L(input params), N_k), fp64."""
    lib = _load()
    x = _x32(x)
    n, d = x.shape
    w, mu, var = _p64(w), _p64(mu), _p64(var)
    k = w.shape[0]
    w2, mu2, v2, nk = np.empty(k), np.empty((k, d)), np.empty((k, d)), np.empty(k)
    L = ctypes.c_double(0.0)
    _check(lib.oracle_em_step(_ptr(x, ctypes.c_float), n, d, k, _ptr(w, ctypes.c_double),
                              _ptr(mu, ctypes.c_double), _ptr(var, ctypes.c_double),
                              float(var_floor), _ptr(w2, ctypes.c_double),
                              _ptr(mu2, ctypes.c_double), _ptr(v2, ctypes.c_double),
                              ctypes.byref(L), _ptr(nk, ctypes.c_double)))
    return w2, mu2, v2, L.value, nk


def loglik(x, w, mu, var, per_row: bool = False):
    """Total log-likelihood sum_n lse_n (and the per-row values if asked)."""
    lib = _load()
    x = _x32(x)
    n, d = x.shape
    w, mu, var = _p64(w), _p64(mu), _p64(var)
    rows = np.empty(n) if per_row else None
    L = ctypes.c_double(0.0)
    _check(lib.oracle_loglik(_ptr(x, ctypes.c_float), n, d, w.shape[0], _ptr(w, ctypes.c_double),
                             _ptr(mu, ctypes.c_double), _ptr(var, ctypes.c_double),
                             ctypes.byref(L), _ptr(rows, ctypes.c_double) if per_row else None))
    return (L.value, rows) if per_row else L.value


def logdensity(x, w, mu, var) -> np.ndarray:
    """The n x K matrix of log(w_k N(x_n | mu_k, var_k)) for a few rows."""
    lib = _load()
    x = _x32(x)
    n, d = x.shape
    w, mu, var = _p64(w), _p64(mu), _p64(var)
    out = np.empty((n, w.shape[0]))
    _check(lib.oracle_logdensity(_ptr(x, ctypes.c_float), n, d, w.shape[0],
                                 _ptr(w, ctypes.c_double), _ptr(mu, ctypes.c_double),
                                 _ptr(var, ctypes.c_double), _ptr(out, ctypes.c_double)))
    return out


def kmeans_step(x, c):
    """One Lloyd step from centroids c: (c', assignment int32, inertia of c, N_k)."""
    lib = _load()
    x = _x32(x)
    n, d = x.shape
    c = _p64(c)
    k = c.shape[0]
    c2, z, nk = np.empty((k, d)), np.empty(n, np.int32), np.empty(k)
    inertia = ctypes.c_double(0.0)
    _check(lib.oracle_kmeans_step(_ptr(x, ctypes.c_float), n, d, k, _ptr(c, ctypes.c_double),
                                  _ptr(c2, ctypes.c_double), _ptr(z, ctypes.c_int32),
                                  ctypes.byref(inertia), _ptr(nk, ctypes.c_double)))
    return c2, z, inertia.value, nk


def topm(x, w, mu, var, m: int):
    """Top-m components per row by responsibility: (idx int32, resp, gap)."""
    lib = _load()
    x = _x32(x)
    n, d = x.shape
    w, mu, var = _p64(w), _p64(mu), _p64(var)
    idx = np.empty((n, m), dtype=np.int32)
    resp = np.empty((n, m))
    gap = np.empty(n)
    _check(lib.oracle_topm(_ptr(x, ctypes.c_float), n, d, w.shape[0], _ptr(w, ctypes.c_double),
                           _ptr(mu, ctypes.c_double), _ptr(var, ctypes.c_double), int(m),
                           _ptr(idx, ctypes.c_int32), _ptr(resp, ctypes.c_double),
                           _ptr(gap, ctypes.c_double)))
    return idx, resp, gap


def fit(x, w, mu, var, var_floor: float = 1e-6, iters: int = 10, tol: float = 0.0,
        param_dtype=np.float64):
    """Run EM. Returns (w, mu, var, history) with history[t] = L(theta_t).

    Stops early only when tol > 0 and L(theta_t) - L(theta_{t-1}) <
    tol * |L(theta_t)|; the parameters returned are those after the last
    step taken.

    ``param_dtype=np.float32`` rounds the parameters to fp32 after every step
    (the precision in which a caller that stores fp32 parameters carries them
    from one step to the next); each step's arithmetic stays fp64. Comparing
    that trajectory with the fp64 one measures how much EM's own dynamics
    amplify a one-ulp perturbation of the parameters over the iterations.
    """
    hist = []
    for _ in range(iters):
        w2, mu2, v2, L, _ = em_step(x, w, mu, var, var_floor)
        hist.append(L)
        if param_dtype is not np.float64:
            w2, mu2, v2 = (np.asarray(a, dtype=param_dtype).astype(np.float64) for a in (w2, mu2, v2))
        w, mu, var = w2, mu2, v2
        if tol > 0 and len(hist) >= 2 and hist[-1] - hist[-2] < tol * abs(hist[-1]):
            break
    return w, mu, var, np.array(hist)


def brute_em_step(x, w, mu, var, var_floor: float = 1e-6):
    """Materialised N x K EM step in numpy fp64 (tiny inputs only).

    Same definition as ``em_step``, written independently: responsibilities
    are formed as a full matrix and the variance is the two-pass weighted
    variance about the new mean.
    """
    X = _x32(x).astype(np.float64)
    w, mu, var = _p64(w), _p64(mu), _p64(var)
    n, d = X.shape
    with np.errstate(divide="ignore"):
        logw = np.log(w)
    diff = X[:, None, :] - mu[None, :, :]  # N x K x D
    quad = (diff * diff / var[None, :, :]).sum(axis=2)
    logdet = np.log(var).sum(axis=1)
    ell = logw[None, :] - 0.5 * (d * np.log(2.0 * np.pi) + logdet[None, :] + quad)
    m = ell.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(ell - m).sum(axis=1))
    r = np.exp(ell - lse[:, None])  # the N x K responsibility matrix
    nk = r.sum(axis=0)
    w2 = nk / n
    mu2 = mu.copy()
    v2 = var.copy()
    live = nk > 0
    mu2[live] = (r[:, live].T @ X) / nk[live, None]
    for j in np.nonzero(live)[0]:
        dev = X - mu2[j]
        v2[j] = np.maximum((r[:, j, None] * dev * dev).sum(axis=0) / nk[j], var_floor)
    w2[~live] = 0.0
    return w2, mu2, v2, float(lse.sum()), nk, r


def ivf_lists(idx, resp, k: int, min_resp: float = 0.0):
    """Inverted lists from top-m soft assignments.

    idx (N, m) int component ids and resp (N, m) responsibilities, most
    responsible first (as ``topm`` returns them). Row n is stored in the list
    of idx[n, 0] and, for j >= 1, in the list of idx[n, j] when
    resp[n, j] >= min_resp (the border-vector multi-assignment of the IVF
    coarse quantizer; "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
    Clustering", abstract and section 1). Entries whose id is outside [0, k)
    are not stored. Each list holds its rows in increasing order.

    Returns (offsets int64 (k + 1,), rows int32, values float32): list c is
    rows[offsets[c]:offsets[c + 1]], with the responsibilities alongside.
    """
    idx = np.asarray(idx)
    resp = np.asarray(resp, dtype=np.float32)
    n, m = idx.shape
    row = np.repeat(np.arange(n, dtype=np.int64), m)
    col = np.tile(np.arange(m), n)
    key = idx.reshape(-1).astype(np.int64)
    val = resp.reshape(-1)
    keep = (key >= 0) & (key < k) & ((col == 0) | (val >= np.float32(min_resp)))
    key, row, val = key[keep], row[keep], val[keep]
    # a stable sort by list id keeps each list's rows in entry (= row) order
    order = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=k)
    offsets = np.zeros(k + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return offsets, row[order].astype(np.int32), val[order]
