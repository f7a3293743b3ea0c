"""Write the oracle's end-to-end EM results for the two long parity cases.

Test infrastructure: this script calls only the fp64 CPU oracle (oracle/)
and the seeded input generator, never the HIP library. It fits EM from the
seeded initial parameters on a row prefix of two workloads and stores what
the GPU end-to-end tests compare against:

* bf16_large: the first 1,000,000 rows (D = 128, K = 4096, bf16 data),
  5 iterations;
* wide: the first 200,000 rows (D = 768, K = 16384), 3 iterations, then the
  top-2 components (by responsibility) of 512 seeded rows under the fitted
  parameters (the border-vector multi-assignment pass).

Stored per case (tests/golden/endtoend_<case>.npz): the log-likelihood
history, every weight, the means and variances of a seeded sample of
components (all of them would be hundreds of MB), and for the wide case the
top-2 indices, responsibilities and the oracle's margin l_(2) - l_(3).

Usage: python tests/golden/make_endtoend_golden.py [bf16_large|wide ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from gmm_em_amd import datagen as dg  # noqa: E402
from oracle import oracle  # noqa: E402

CASES = {
    # name: (workload, prefix rows, iterations, sampled components, top-m rows)
    "bf16_large": ("bf16_large", 1_000_000, 5, 64, 0),
    "wide": ("wide", 200_000, 3, 32, 512),
}


def path(case: str) -> str:
    return os.path.join(HERE, f"endtoend_{case}.npz")


def make(case: str) -> None:
    wl, n, iters, ncomp, ntop = CASES[case]
    W = dg.WORKLOADS[wl]
    t0 = time.time()
    x = dg.rows(W, n)
    w0, m0, v0 = dg.init_params(W, x)
    w, mu, var, hist = oracle.fit(x, w0, m0, v0, W.var_floor, iters)
    rng = np.random.Generator(np.random.PCG64(7000 + W.index))
    comps = np.sort(rng.choice(W.k, size=ncomp, replace=False))
    out = dict(workload=wl, n=n, iters=iters, hist=hist, weights=w, comps=comps,
               means=mu[comps], variances=var[comps])
    if ntop:
        rows = np.sort(rng.choice(n, size=ntop, replace=False))
        idx, resp, gap = oracle.topm(x[rows], w, mu, var, 2)
        out.update(top_rows=rows, top_idx=idx, top_resp=resp, top_gap=gap)
    np.savez_compressed(path(case), **out)
    print(f"{case}: {n} rows, {iters} iterations, {time.time() - t0:.0f} s, "
          f"{oracle.num_threads()} threads -> {path(case)}", flush=True)


if __name__ == "__main__":
    for c in sys.argv[1:] or list(CASES):
        make(c)
