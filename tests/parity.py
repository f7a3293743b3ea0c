"""Comparison helpers for GPU-vs-oracle parity tests (test infrastructure).

Tolerances follow the stated parity bar for this method: means, variances and
weights within 1e-4 relative for fp32 data (5e-3 for bf16 data) and the total
log-likelihood within 1e-5 relative. "Relative" is read per component:
  mean:     max_d |dmu_kd| / max(max_d |mu_kd|, max_d sqrt(var_kd))
  variance: max_d |dvar_kd| / var_kd
  weight:   |dw_k| / max(w_k, 1/N)
over components whose oracle responsibility mass N_k >= 1.
"""
import numpy as np


def param_errors(gpu, ref, nk, n):
    """gpu/ref = (w, mu, var); returns dict of max relative errors (live comps)."""
    gw, gmu, gv = (np.asarray(a, dtype=np.float64) for a in gpu)
    rw, rmu, rv = (np.asarray(a, dtype=np.float64) for a in ref)
    live = np.asarray(nk) >= 1.0
    scale = np.maximum(np.abs(rmu).max(axis=1), np.sqrt(rv).max(axis=1))
    emu = np.abs(gmu - rmu).max(axis=1) / scale
    ev = (np.abs(gv - rv) / rv).max(axis=1)
    ew = np.abs(gw - rw) / np.maximum(rw, 1.0 / n)
    out = {
        "mu": float(emu[live].max()) if live.any() else 0.0,
        "var": float(ev[live].max()) if live.any() else 0.0,
        "w": float(ew[live].max()) if live.any() else 0.0,
        "n_live": int(live.sum()),
    }
    # dead components (oracle mass exactly 0): frozen mean/variance, weight 0
    dead = np.asarray(nk) == 0.0
    out["dead_ok"] = bool(np.all(gw[dead] == 0.0) and np.array_equal(gmu[dead], rmu[dead].astype(np.float32))
                          ) if dead.any() else True
    return out


def assert_params_close(gpu, ref, nk, n, tol=1e-4, what=""):
    e = param_errors(gpu, ref, nk, n)
    msg = f"{what} errors {e} (tol {tol})"
    assert e["mu"] <= tol and e["var"] <= tol and e["w"] <= tol, msg
    assert e["dead_ok"], msg
    return e


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)
