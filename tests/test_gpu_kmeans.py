"""GPU parity of the k-means (Lloyd) mode against the oracle's Lloyd step.

The GPU's distances use the expanded form about a per-dimension shift, in
fp64 or on exact int8 slices (integer-valued data), the oracle's the direct
sum of squared differences in fp64. Where the two
nearest centroids of a row are within rounding of each other the two sides
may pick different ones; such a row is accepted when the GPU's choice is
within the fp64 rounding bound of the best distance, and the clusters it
touches are left out of the centroid comparison. Everything else is compared
element by element: assignments exactly, centroids to 1e-4 relative (per
cluster, against max(max_d |c_kd|, 1)), inertia to 1e-5 relative. Empty
clusters keep their centroid bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gmm_em_amd import datagen as dg  # noqa: E402
from oracle import oracle  # noqa: E402
from tests.parity import rel  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    from gmm_em_amd import ops as o

    return o


def _xt(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _dist2(xf, c):
    """Row-wise fp64 squared distance between matching rows of xf and c."""
    diff = xf.astype(np.float64) - c.astype(np.float64)
    return np.einsum("nd,nd->n", diff, diff)


def _near_tie_rows(x, c_in, z_gpu, z_ref):
    """Rows where the assignments differ; asserts each is a rounding-level tie."""
    bad = np.nonzero(z_gpu != z_ref)[0]
    if bad.size == 0:
        return bad
    xf = dg.as_f32(x[bad]).astype(np.float64)
    dgpu = _dist2(xf, c_in[z_gpu[bad]])
    dref = _dist2(xf, c_in[z_ref[bad]])
    scale = (np.einsum("nd,nd->n", xf, xf) + np.einsum("nd,nd->n", c_in[z_gpu[bad]], c_in[z_gpu[bad]])
             + np.einsum("nd,nd->n", c_in[z_ref[bad]], c_in[z_ref[bad]]) + 1.0)
    assert np.all(z_gpu[bad] >= 0) and np.all(z_gpu[bad] < len(c_in))
    assert np.all(dgpu - dref <= 1e-12 * scale), (bad[:5], dgpu[:5], dref[:5])
    assert bad.size <= max(3, len(z_gpu) // 10000), f"{bad.size} differing assignments"
    return bad


def _check_step(x, c_in, c_gpu, z_gpu, inertia_gpu, label, tol=1e-4):
    """One GPU Lloyd step (from c_in) against the oracle's; returns the worst error."""
    c2, z, inertia, nk = oracle.kmeans_step(x, c_in)
    bad = _near_tie_rows(x, c_in, z_gpu, z)
    assert rel(inertia_gpu, inertia) <= 1e-5, f"{label}: inertia {inertia_gpu} vs {inertia}"
    touched = np.zeros(len(c_in), bool)
    touched[z_gpu[bad]] = True
    touched[z[bad]] = True
    live = (nk > 0) & ~touched
    scale = np.maximum(np.abs(c2).max(axis=1), 1.0)
    err = np.abs(c_gpu.astype(np.float64) - c2).max(axis=1) / scale
    worst = float(err[live].max()) if live.any() else 0.0
    assert worst <= tol, f"{label}: centroid error {worst}"
    dead = (nk == 0) & ~touched
    assert np.array_equal(c_gpu[dead], c_in[dead].astype(np.float32)), f"{label}: empty cluster moved"
    return worst, int(bad.size)


def _run(ops, x, c0, steps, label, tol=1e-4, path=None):
    xt = _xt(x)
    c = torch.from_numpy(np.ascontiguousarray(c0, dtype=np.float32)).to(DEV)
    ws = ops.workspace(x.shape[1], len(c0), DEV)
    prev = np.inf
    for t in range(steps):
        c_in = c.cpu().numpy().astype(np.float64)
        inertia, z = ops.kmeans_step(xt, c, ws=ws)
        torch.cuda.synchronize()
        I = inertia.item()
        worst, nbad = _check_step(x, c_in, c.cpu().numpy(), z.cpu().numpy(), I, f"{label} step {t}", tol)
        print(f"{label} step {t}: centroid err {worst:.2e}, tie rows {nbad}, inertia {I:.6e}")
        if path is not None:  # which distance arithmetic the device chose
            got = ops.estep_arithmetic(ws, DEV)
            assert got == path, f"{label} step {t}: distance arithmetic {got}, expected {path}"
        # Lloyd never increases the inertia (up to the fp32 rounding of c)
        assert I <= prev * (1 + 1e-7) + 1e-9
        prev = I
    assert ops.device_status(ws, DEV) == ops.GMM_OK


@pytest.mark.parametrize("n,d,k,seed", [(1000, 16, 8, 1),       # one tile of components
                                         (4999, 96, 100, 2),     # ragged rows, K not a tile multiple
                                         (3000, 37, 130, 3),     # odd D, K just past a 128-group
                                         (9000, 128, 50, 4),     # the widest narrow padding
                                         (777, 5, 300, 5)])      # many clusters for few rows
def test_kmeans_per_step_ragged(ops, n, d, k, seed):
    x, _, _ = dg.custom(n, d, k, seed=seed)
    rng = np.random.default_rng(seed)
    c0 = x[rng.choice(n, k, replace=False)].astype(np.float32)
    # real-valued data: the distances run in fp64
    _run(ops, x, c0, 4, f"kmeans n={n} d={d} k={k}", path=ops.GMM_ESTEP_FP64)


@pytest.mark.parametrize("n,d,k,seed", [(1000, 16, 8, 11), (4999, 96, 100, 12), (3000, 37, 130, 13),
                                         (9000, 128, 50, 14), (777, 5, 300, 15)])
def test_kmeans_int8_integer_data(ops, n, d, k, seed):
    # integer-valued data in [0, 120] (one digit for a, two for a^2): the
    # distances run on exact int8 slices, the same shapes as above
    x, _, _ = dg.custom(n, d, k, seed=seed)
    x = np.clip(np.rint(x * 8.0 + 40.0), 0, 120).astype(np.float32)
    rng = np.random.default_rng(seed)
    c0 = x[rng.choice(n, k, replace=False)].astype(np.float32)
    _run(ops, x, c0, 4, f"kmeans int8 n={n} d={d} k={k}", path=ops.GMM_ESTEP_INT8_SLICES)


def test_kmeans_bf16_per_step(ops):
    x, _, _ = dg.custom(3000, 64, 40, seed=7, dtype="bf16")
    xf = dg.as_f32(x)
    c0 = xf[np.random.default_rng(7).choice(3000, 40, replace=False)]
    _run(ops, x, c0, 3, "kmeans bf16")


def test_kmeans_empty_and_duplicate_centroids(ops):
    x, _, _ = dg.custom(2000, 24, 6, seed=9)
    c0 = x[:8].astype(np.float32).copy()
    c0[3] = c0[1]           # exact duplicate: every tie goes to the smaller index
    c0[5] = 1.0e4           # far from every row: an empty cluster
    xt = _xt(x)
    c = torch.from_numpy(c0.copy()).to(DEV)
    inertia, z = ops.kmeans_step(xt, c)
    torch.cuda.synchronize()
    zg, cg = z.cpu().numpy(), c.cpu().numpy()
    assert not np.any(zg == 3) and not np.any(zg == 5)
    assert np.array_equal(cg[3], c0[3]) and np.array_equal(cg[5], c0[5])
    _check_step(x, c0.astype(np.float64), cg, zg, inertia.item(), "empty/duplicate")


def test_kmeans_without_assignment_output_is_identical(ops):
    # without an assignment array the chunk's assignments live in the
    # workspace scratch; the results must not change (bitwise)
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 50_000)
    _, m0, _ = dg.init_params(W, x)
    xt = _xt(x)
    outs = []
    for assign in (True, False):
        c = torch.from_numpy(m0.copy()).to(DEV)
        inertia, _ = ops.kmeans_step(xt, c, assign=assign)
        torch.cuda.synchronize()
        outs.append((inertia.item(), c.cpu().numpy()))
    assert outs[0][0] == outs[1][0]
    assert np.array_equal(outs[0][1], outs[1][1])


def test_kmeans_invalid_centroid_reports_params(ops):
    x, _, _ = dg.custom(500, 8, 4, seed=3)
    c0 = x[:4].astype(np.float32).copy()
    c0[2, 5] = np.nan
    c = torch.from_numpy(c0).to(DEV)
    ws = ops.workspace(8, 4, DEV)
    inertia, _ = ops.kmeans_step(_xt(x), c, ws=ws)
    assert ops.device_status(ws, DEV) == ops.GMM_E_PARAMS
    assert np.isnan(inertia.item()) and np.all(np.isnan(c.cpu().numpy()))


def test_kmeans_descriptor_prefix_per_step(ops):
    # the headline workload's shape (D=96, K=1024, integer-valued data) on a
    # 60,000-row prefix, from the seeded initial means
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 60_000)
    _, m0, _ = dg.init_params(W, x)
    _run(ops, x, m0, 2, "kmeans descriptor prefix", path=ops.GMM_ESTEP_INT8_SLICES)


def test_kmeans_descriptor_full_size(ops):
    # N = 10,000,000 rows (three row chunks), D = 96, K = 1024. Assignments
    # are checked against the oracle on sampled rows (the ragged tail
    # included); the update and the inertia are checked for every cluster
    # through the oracle's single-cluster step over the rows the GPU put in
    # that cluster, whose result is their mean and summed squared distance.
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W)
    _, m0, _ = dg.init_params(W, x)
    xt = _xt(x)
    c = torch.from_numpy(m0.copy()).to(DEV)
    ws = ops.workspace(W.d, W.k, DEV)
    inertia, z = ops.kmeans_step(xt, c, ws=ws)
    torch.cuda.synchronize()
    assert ops.estep_arithmetic(ws, DEV) == ops.GMM_ESTEP_INT8_SLICES
    zg, cg, I = z.cpu().numpy(), c.cpu().numpy(), inertia.item()
    del xt
    rng = np.random.default_rng(77)
    pick = np.sort(rng.choice(len(x), 4000, replace=False))
    pick[-1] = len(x) - 1
    _, zr, _, _ = oracle.kmeans_step(x[pick], m0)
    _near_tie_rows(x[pick], m0.astype(np.float64), zg[pick], zr)
    order = np.argsort(zg, kind="stable")
    bounds = np.searchsorted(zg[order], np.arange(W.k + 1))
    total, worst = 0.0, 0.0
    for k in range(W.k):
        rows = order[bounds[k]:bounds[k + 1]]
        if rows.size == 0:
            assert np.array_equal(cg[k], m0[k])
            continue
        ck, _, ik, _ = oracle.kmeans_step(x[rows], m0[k:k + 1])
        total += ik
        e = np.abs(cg[k].astype(np.float64) - ck[0]).max() / max(np.abs(ck[0]).max(), 1.0)
        worst = max(worst, e)
    print(f"kmeans descriptor full: centroid err {worst:.2e}, inertia {I:.9e} vs {total:.9e}")
    assert worst <= 1e-4
    assert rel(I, total) <= 1e-5


# ---------------------------------------------------------------------------
# Wide rows (padded dimension 256..768): the wide distance pass and the
# per-slice k-means statistics.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,d,k,seed", [(3000, 300, 40, 21),    # padded 384
                                         (5000, 768, 24, 22),    # padded 768, two row chunks
                                         (2500, 513, 70, 23)])   # padded 640, ragged dims
def test_kmeans_wide_per_step(ops, n, d, k, seed):
    x, _, _ = dg.custom(n, d, k, seed=seed)
    rng = np.random.default_rng(seed)
    c0 = x[rng.choice(n, k, replace=False)].astype(np.float32)
    _run(ops, x, c0, 3, f"kmeans wide n={n} d={d} k={k}")


def test_kmeans_wide_bf16(ops):
    x, _, _ = dg.custom(2000, 256, 30, seed=24, dtype="bf16")
    xf = dg.as_f32(x)
    c0 = xf[np.random.default_rng(24).choice(2000, 30, replace=False)]
    _run(ops, x, c0, 2, "kmeans wide bf16")


def test_kmeans_wide_workload_prefix(ops):
    # the wide many-component workload (D = 768, K = 16384) on a 20,000-row
    # prefix, from its seeded initial means
    W = dg.WORKLOADS["wide"]
    x = dg.rows(W, 20_000)
    _, m0, _ = dg.init_params(W, x)
    _run(ops, x, m0, 1, "kmeans wide workload prefix")


def test_kmeans_fit_matches_chained_oracle_steps(ops):
    # five Lloyd steps end to end from the same centroids on both sides, and
    # the early stop on the relative inertia decrease
    x, _, _ = dg.custom(4000, 12, 10, seed=31)
    c0 = x[np.random.default_rng(31).choice(4000, 10, replace=False)].astype(np.float32)
    c = torch.from_numpy(c0.copy()).to(DEV)
    hist, done = ops.kmeans_fit(_xt(x), c, max_iter=5)
    torch.cuda.synchronize()
    assert done == 5
    ref = c0.astype(np.float64)
    rhist = []
    for _ in range(5):
        ref, _, inertia, _ = oracle.kmeans_step(x, ref.astype(np.float32).astype(np.float64))
        rhist.append(inertia)
    h = hist.cpu().numpy()
    assert np.all(np.abs(h - rhist) / np.array(rhist) <= 1e-5), (h, rhist)
    g = c.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g - ref) / np.maximum(np.abs(ref).max(axis=1, keepdims=True), 1.0)) <= 1e-4
    # with a tolerance the loop stops once the inertia stops improving
    c2 = torch.from_numpy(c0.copy()).to(DEV)
    _, done2 = ops.kmeans_fit(_xt(x), c2, max_iter=200, tol=1e-9)
    assert 1 <= done2 < 200
