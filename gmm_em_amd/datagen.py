"""Seeded synthetic inputs for the fused diagonal-GMM EM step.

This module only draws inputs: planted mixtures, the data rows sampled from
them, and the initial parameters an EM run starts from. It performs none of
the EM arithmetic, so both the fp64 CPU oracle and the HIP path can consume
its arrays without sharing any computation.

The workloads stand in for the unnamed ANN datasets and benchmark workloads
that the Flash-GMM pages measure on ("Flash-GMM: A Memory-Efficient Kernel for
Scalable Soft Clustering", section 3, Table 1 and Figure 1): none of those are
available, so each workload is a planted diagonal Gaussian mixture with the
shape, value range and weight profile stated in ``WORKLOADS``.

Determinism rules (bit-identical on any machine, chunk-parallel):

* planted parameters come from ``Generator(PCG64(1000 + i))`` in the order
  means, spread (standard deviation or variance), weights;
* rows are drawn in fixed chunks of ``CHUNK_ROWS`` rows; chunk ``c`` uses
  ``Generator(PCG64(SeedSequence([1000 + i, c])))`` and draws labels
  ``z ~ Cat(w)`` first, then ``eps ~ N(0, I)``; ``x = mu*_z + sd*_z * eps``
  is formed in fp64 and only then rounded to the storage type;
* the initial means are ``K`` distinct rows chosen by
  ``Generator(PCG64(2000 + i)).choice(N, K, replace=False)``; initial
  variances are 1 and initial weights 1/K.

A row prefix of a workload is simply its first rows, so a parity case on the
first ``n`` rows of a large workload sees exactly those rows.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 1 << 20


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, generator recipe and iteration count."""

    key: str
    index: int  # seeds are 1000 + index (data) and 2000 + index (init)
    n: int
    d: int
    k: int
    dtype: str  # storage type of X: "f32" or "bf16"
    iters: int
    recipe: str
    var_floor: float = 1e-6


WORKLOADS = {
    # 8 planted components, means ~ N(0, 4^2 I), per-dim variances ~ U[0.5, 2],
    # Dirichlet(1) weights; small enough for the oracle to run every iteration.
    "tiny": Workload("tiny", 1, 10_000, 16, 8, "f32", 20, "tiny"),
    # Embedding-like: unit-norm means, per-dim sd ~ U[0.05, 0.2], Dirichlet(1).
    "embed": Workload("embed", 2, 1_000_000, 128, 256, "f32", 10, "embed"),
    # Non-negative integer descriptors: means ~ U[0, 100]^D, sd ~ U[2, 10],
    # x clipped at 0 and rounded to integers, Zipf(1.1) weights.
    "descriptor": Workload("descriptor", 3, 10_000_000, 96, 1024, "f32", 10, "descriptor"),
    # Large N with bf16 storage: unit-norm means, sd ~ U[0.03, 0.15],
    # Dirichlet(0.5) weights.
    "bf16_large": Workload("bf16_large", 4, 50_000_000, 128, 4096, "bf16", 5, "bf16_large"),
    # Wide and many-component: unit-norm means, sd ~ U[0.01, 0.05], uniform
    # weights; also used for the top-2 border-vector assignment.
    "wide": Workload("wide", 5, 5_000_000, 768, 16384, "f32", 3, "wide"),
}


@dataclasses.dataclass
class Planted:
    """Planted mixture: weights (K,), means (K, D), standard deviations (K, D)."""

    weights: np.ndarray
    means: np.ndarray
    sds: np.ndarray


def _unit_rows(a: np.ndarray) -> np.ndarray:
    return a / np.linalg.norm(a, axis=1, keepdims=True)


def planted(w: Workload) -> Planted:
    """Draw the planted mixture of a workload (fp64)."""
    rng = np.random.Generator(np.random.PCG64(1000 + w.index))
    K, D = w.k, w.d
    if w.recipe == "tiny":
        means = rng.normal(0.0, 4.0, size=(K, D))
        variances = rng.uniform(0.5, 2.0, size=(K, D))  # the recipe draws variances
        sds = np.sqrt(variances)
        weights = rng.dirichlet(np.ones(K))
    elif w.recipe == "embed":
        means = _unit_rows(rng.standard_normal((K, D)))
        sds = rng.uniform(0.05, 0.2, size=(K, D))
        weights = rng.dirichlet(np.ones(K))
    elif w.recipe == "descriptor":
        means = rng.uniform(0.0, 100.0, size=(K, D))
        sds = rng.uniform(2.0, 10.0, size=(K, D))
        ranks = np.arange(1, K + 1, dtype=np.float64)
        weights = ranks ** -1.1
        weights /= weights.sum()
    elif w.recipe == "bf16_large":
        means = _unit_rows(rng.standard_normal((K, D)))
        sds = rng.uniform(0.03, 0.15, size=(K, D))
        weights = rng.dirichlet(np.full(K, 0.5))
    elif w.recipe == "wide":
        means = _unit_rows(rng.standard_normal((K, D)))
        sds = rng.uniform(0.01, 0.05, size=(K, D))
        weights = np.full(K, 1.0 / K)
    else:  # pragma: no cover - closed set
        raise ValueError(w.recipe)
    return Planted(weights=weights, means=means, sds=sds)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Rounding is done once, directly
    from fp64, on the bit pattern: bfloat16 keeps 7 of fp64's 52 fraction
    bits and fp64's exponent range covers bfloat16's, so for finite inputs in
    bfloat16's normal range (all this module produces) adding half an ulp
    with the tie-to-even bit and truncating is exact rounding.
    """
    u = np.ascontiguousarray(a, dtype=np.float64).view(np.uint64)
    drop = np.uint64(45)  # 52 - 7 fraction bits dropped
    lsb = (u >> drop) & np.uint64(1)
    # add just under half an ulp of the kept precision (2^44 - 1), plus the
    # kept lsb so that exact ties round to even, then truncate
    u = (u + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    # the rounded value is exactly representable in fp32, so this cast is exact
    f = u.view(np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _chunk(w: Workload, p: Planted, c: int, rows: int, need: int) -> np.ndarray:
    # labels are drawn for the whole chunk, so the normal stream that follows
    # starts at the same place whatever prefix is asked for; the normals are
    # drawn in row-major order, so the first `need` rows are a prefix of the
    # whole chunk's draw
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + w.index, c])))
    z = rng.choice(w.k, size=rows, p=p.weights)[:need]
    eps = rng.standard_normal((need, w.d))
    x = p.means[z] + p.sds[z] * eps
    if w.recipe == "descriptor":
        x = np.maximum(np.rint(x), 0.0)  # rint rounds half to even; then clip at +0
    if w.dtype == "bf16":
        return f64_to_bf16_bits(x)
    return x.astype(np.float32)


def rows(w: Workload, n: int | None = None, threads: int | None = None) -> np.ndarray:
    """The first ``n`` rows (default all N) of a workload's data matrix.

    Returns an (n, D) array: float32, or uint16 bfloat16 bit patterns for a
    bf16 workload. Chunks are drawn in parallel threads; the result does not
    depend on the thread count.
    """
    n = w.n if n is None else int(n)
    if n < 0 or n > w.n:
        raise ValueError(f"row count {n} outside [0, {w.n}]")
    p = planted(w)
    out = np.empty((n, w.d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    nchunks = (n + CHUNK_ROWS - 1) // CHUNK_ROWS

    def work(c: int) -> None:
        lo = c * CHUNK_ROWS
        hi = min(n, lo + CHUNK_ROWS)
        full = min(CHUNK_ROWS, w.n - lo)  # chunk content never depends on n
        out[lo:hi] = _chunk(w, p, c, full, hi - lo)

    threads = threads or min(16, os.cpu_count() or 1)
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def labels(w: Workload, n: int | None = None) -> np.ndarray:
    """Planted component label of each of the first ``n`` rows (int64)."""
    n = w.n if n is None else int(n)
    p = planted(w)
    out = np.empty(n, dtype=np.int64)
    for c in range((n + CHUNK_ROWS - 1) // CHUNK_ROWS):
        lo = c * CHUNK_ROWS
        hi = min(n, lo + CHUNK_ROWS)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + w.index, c])))
        out[lo:hi] = rng.choice(w.k, size=min(CHUNK_ROWS, w.n - lo), p=p.weights)[: hi - lo]
    return out


def as_f32(x: np.ndarray) -> np.ndarray:
    """Data rows as fp32 (bf16 bit patterns are widened exactly)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def init_params(w: Workload, x: np.ndarray, n_total: int | None = None):
    """Initial (weights, means, variances) as fp32 arrays.

    Means are K distinct rows of ``x`` picked with a seeded draw over the
    ``n_total`` rows the run uses (default: all rows of ``x``); variances are
    1 and weights 1/K. Every value is exact in fp32.
    """
    n_total = x.shape[0] if n_total is None else n_total
    if n_total < w.k:
        raise ValueError("need at least K rows to seed K distinct means")
    rng = np.random.Generator(np.random.PCG64(2000 + w.index))
    idx = rng.choice(n_total, size=w.k, replace=False)
    means = np.ascontiguousarray(as_f32(x[idx]), dtype=np.float32)
    variances = np.ones((w.k, w.d), dtype=np.float32)
    weights = np.full(w.k, 1.0 / w.k, dtype=np.float32)
    return weights, means, variances


def custom(n: int, d: int, k: int, seed: int, spread: float = 4.0, sd_lo: float = 0.5,
           sd_hi: float = 2.0, dtype: str = "f32"):
    """A small ad-hoc planted mixture for tests of arbitrary shape.

    Returns (x, planted) with x of shape (n, d). Means ~ N(0, spread^2 I),
    per-dim sd ~ U[sd_lo, sd_hi], Dirichlet(1) weights, all from
    ``Generator(PCG64(seed))``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    means = rng.normal(0.0, spread, size=(k, d))
    sds = rng.uniform(sd_lo, sd_hi, size=(k, d))
    weights = rng.dirichlet(np.ones(k))
    z = rng.choice(k, size=n, p=weights)
    x = means[z] + sds[z] * rng.standard_normal((n, d))
    x = f64_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    return x, Planted(weights=weights, means=means, sds=sds), z
