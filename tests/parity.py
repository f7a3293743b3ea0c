"""Comparison helpers for GPU-vs-oracle parity tests (test infrastructure).

Tolerances follow the stated parity bar for this method: means, variances and
weights within 1e-4 relative for fp32 data (5e-3 for bf16 data) and the total
log-likelihood within 1e-5 relative. "Relative" is read per component:
  mean:     max_d |dmu_kd| / max(max_d |mu_kd|, max_d sqrt(var_kd))
  variance: max_d |dvar_kd| / var_kd
  weight:   |dw_k| / max(w_k, 1/N)
Components are split by the oracle's responsibility mass N_k:
  N_k >= 1      ("live"): the bar above;
  0 < N_k < 1   ("tiny"): the weighted mean of far tails is ill-conditioned,
                so these are checked to 1e-2 and their count is reported;
  N_k == 0      ("dead"): the GPU must also give weight 0 and keep the
                component's mean.
A component that the GPU kills (weight exactly 0) while the oracle keeps it
(N_k > 0) is counted separately ("killed") and must not occur.
"""
import numpy as np

TINY_TOL = 1e-2


def _errors(gw, gmu, gv, rw, rmu, rv, n):
    scale = np.maximum(np.abs(rmu).max(axis=1), np.sqrt(rv).max(axis=1))
    emu = np.abs(gmu - rmu).max(axis=1) / scale
    ev = (np.abs(gv - rv) / rv).max(axis=1)
    ew = np.abs(gw - rw) / np.maximum(rw, 1.0 / n)
    return emu, ev, ew


def param_errors(gpu, ref, nk, n):
    """gpu/ref = (w, mu, var); returns a dict of max relative errors per class."""
    gw, gmu, gv = (np.asarray(a, dtype=np.float64) for a in gpu)
    rw, rmu, rv = (np.asarray(a, dtype=np.float64) for a in ref)
    nk = np.asarray(nk, dtype=np.float64)
    emu, ev, ew = _errors(gw, gmu, gv, rw, rmu, rv, n)
    live = nk >= 1.0
    tiny = (nk > 0.0) & (nk < 1.0)
    dead = nk == 0.0

    def worst(e, sel):
        return float(e[sel].max()) if sel.any() else 0.0

    out = {
        "mu": worst(emu, live), "var": worst(ev, live), "w": worst(ew, live),
        "n_live": int(live.sum()),
        "n_tiny": int(tiny.sum()),
        "tiny_worst": max(worst(emu, tiny), worst(ev, tiny), worst(ew, tiny)),
        "n_dead": int(dead.sum()),
        "killed": int(np.sum((nk > 0.0) & (gw == 0.0))),
    }
    out["dead_ok"] = bool(np.all(gw[dead] == 0.0) and
                          np.array_equal(gmu[dead].astype(np.float32), rmu[dead].astype(np.float32))
                          ) if dead.any() else True
    return out


def assert_params_close(gpu, ref, nk, n, tol=1e-4, what=""):
    e = param_errors(gpu, ref, nk, n)
    msg = f"{what} errors {e} (tol {tol})"
    assert e["mu"] <= tol and e["var"] <= tol and e["w"] <= tol, msg
    assert e["tiny_worst"] <= TINY_TOL, msg
    assert e["killed"] == 0, msg
    assert e["dead_ok"], msg
    return e


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)
