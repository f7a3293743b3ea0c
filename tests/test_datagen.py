"""The seeded input generator: determinism, prefixes and bf16 rounding."""
import numpy as np
import torch

from gmm_em_amd import datagen as dg


def test_rows_deterministic_and_thread_independent():
    W = dg.WORKLOADS["embed"]
    a = dg.rows(W, 5000, threads=1)
    b = dg.rows(W, 5000, threads=4)
    assert a.dtype == np.float32 and a.shape == (5000, 128)
    assert np.array_equal(a, b)


def test_prefix_is_a_prefix_across_chunks():
    W = dg.WORKLOADS["tiny"]
    full = dg.rows(W)
    assert np.array_equal(dg.rows(W, 1234), full[:1234])
    big = dg.WORKLOADS["descriptor"]
    two = dg.rows(big, dg.CHUNK_ROWS + 10)
    assert np.array_equal(two[:100], dg.rows(big, 100))
    assert np.all(two >= 0) and np.array_equal(two, np.rint(two))  # clipped integers


def test_descriptor_labels_follow_zipf_weights():
    W = dg.WORKLOADS["descriptor"]
    z = dg.labels(W, 200_000)
    p = dg.planted(W).weights
    assert p[0] > p[1] > p[-1]
    assert abs((z == 0).mean() - p[0]) < 5 * np.sqrt(p[0] / 200_000)


def test_init_params_are_distinct_rows():
    W = dg.WORKLOADS["tiny"]
    x = dg.rows(W)
    w, mu, var = dg.init_params(W, x)
    assert len({tuple(r) for r in mu}) == W.k
    assert all(any(np.array_equal(r, xr) for xr in x) for r in mu)
    assert np.all(var == 1) and np.allclose(w.sum(), 1)


def test_bf16_rounding_matches_torch_on_fp32_exact_values():
    rng = np.random.default_rng(5)
    v = rng.normal(0, 1, size=100_000).astype(np.float32)
    v[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1.0]  # exact ties
    ours = dg.f64_to_bf16_bits(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(dg.bf16_bits_to_f32(ours),
                          torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_bf16_workload_storage():
    W = dg.WORKLOADS["bf16_large"]
    x = dg.rows(W, 1000)
    assert x.dtype == np.uint16 and x.shape == (1000, 128)
    f = dg.as_f32(x)
    assert np.all(np.isfinite(f)) and np.abs(f).max() < 2
