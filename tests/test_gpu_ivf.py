"""GPU parity of the IVF list construction against the oracle (bit-exact).

The inputs are seeded synthetic top-m arrays (with ids outside [0, k) mixed
in), and the GPU's own top-2 soft assignments of the headline workload; the
same host copy of the arrays goes to both sides. Offsets, row ids and values
must be identical.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gmm_em_amd import datagen as dg  # noqa: E402
from oracle import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    from gmm_em_amd import ops as o

    return o


def _compare(ops, idx, resp, k, tau, label):
    it = torch.from_numpy(np.ascontiguousarray(idx)).to(DEV)
    rt = None if resp is None else torch.from_numpy(np.ascontiguousarray(resp)).to(DEV)
    off, rows, vals = ops.ivf_build(it, rt, k, tau)
    torch.cuda.synchronize()
    r_resp = np.ones(idx.shape, np.float32) if resp is None else resp
    r_tau = -np.inf if resp is None else tau
    roff, rrows, rvals = oracle.ivf_lists(idx, r_resp, k, r_tau)
    np.testing.assert_array_equal(off.cpu().numpy(), roff, err_msg=f"{label}: offsets")
    np.testing.assert_array_equal(rows.cpu().numpy(), rrows, err_msg=f"{label}: rows")
    np.testing.assert_array_equal(vals.cpu().numpy(), rvals, err_msg=f"{label}: values")
    return len(rrows)


def _synthetic(n, m, k, seed, bad=0.01):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, k, size=(n, m)).astype(np.int32)
    if bad > 0 and n > 0:
        mask = rng.uniform(size=(n, m)) < bad
        idx[mask] = rng.choice(np.array([-1, k, k + 7], np.int32), size=int(mask.sum()))
    resp = np.sort(rng.dirichlet(np.ones(m), size=n).astype(np.float32), axis=1)[:, ::-1].copy()
    return idx, resp


@pytest.mark.parametrize("n,m,k,tau,seed", [
    (0, 2, 16, 0.0, 1),          # empty input: all offsets 0
    (1, 1, 1, 0.0, 2),           # one row, one list
    (1000, 2, 8, 0.2, 3),        # one tile, few lists
    (5001, 3, 300, 0.1, 4),      # several tiles with a ragged tail
    (70_000, 4, 1024, 0.05, 5),  # many tiles, headline list count
    (9000, 2, 16384, 0.0, 6),    # the largest list count
    (4000, 2, 2, 0.0, 9),        # two lists: a chunk's lanes share an id, ranks up to 63
    (3000, 3, 1025, 0.0, 10),    # one list past a power of two (11 id bits)
])
def test_ivf_synthetic(ops, n, m, k, tau, seed):
    idx, resp = _synthetic(n, m, k, seed)
    stored = _compare(ops, idx, resp, k, tau, f"n={n} m={m} k={k}")
    print(f"ivf n={n} m={m} k={k} tau={tau}: {stored} entries")


def test_ivf_wide_tiles(ops):
    # n*m*k large enough that the tile size doubles to keep the tiles x K
    # counter matrix within 2^24 entries: 3M rows, top-2, 16384 lists
    idx, resp = _synthetic(3_000_000, 2, 16384, 7)
    assert ops.lib.gmm_ivf_workspace_bytes(3_000_000, 2, 16384) <= (1 << 26) + (1 << 17)
    _compare(ops, idx, resp, 16384, 0.25, "wide tiles")


def test_ivf_without_responsibilities(ops):
    idx, _ = _synthetic(3000, 2, 50, 8)
    _compare(ops, idx, None, 50, 0.0, "no resp")


def test_ivf_from_gpu_topm_descriptor_full(ops):
    # the headline workload (N = 10,000,000, D = 96, K = 1024): top-2 soft
    # assignment on the GPU, then the lists at two thresholds
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W)
    w0, m0, v0 = dg.init_params(W, x)
    xt = torch.from_numpy(x).to(DEV)
    w, mu, var = (torch.from_numpy(a).to(DEV) for a in (w0, m0, v0))
    ws = ops.workspace(W.d, W.k, DEV)
    ops.em_step(xt, w, mu, var, W.var_floor, ws=ws)  # past the initial, almost-hard parameters
    idx, resp = ops.assign_topm(xt, w, mu, var, 2, ws=ws)
    torch.cuda.synchronize()
    del xt
    hi, hr = idx.cpu().numpy(), resp.cpu().numpy()
    for tau in (0.0, 0.1):
        stored = _compare(ops, hi, hr, W.k, tau, f"descriptor tau={tau}")
        print(f"descriptor full top-2 lists, tau={tau}: {stored} entries "
              f"({stored - len(x)} border copies)")
