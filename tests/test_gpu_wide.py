"""GPU parity of the wide path (padded dimension 256..768) against the oracle.

Same conventions as test_gpu_parity: per-step comparisons hand the GPU's fp32
parameters (converted exactly) to the oracle; seeded inputs on both sides.
Shapes cover every wide padded size, ragged row counts across the wide row
chunk (4096 rows), dims that are not multiples of the padding, and the wide
many-component workload (D=768, K=16384) on a row prefix.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gmm_em_amd import datagen as dg  # noqa: E402
from oracle import oracle  # noqa: E402
from tests.parity import assert_params_close, rel  # noqa: E402
from tests.test_gpu_parity import _check_topm, _gpu_step, _host, _per_step, _to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    from gmm_em_amd import ops as o

    return o


def _init(x, k, seed):
    rng = np.random.default_rng(seed)
    n, d = x.shape
    w0 = rng.dirichlet(np.ones(k)).astype(np.float32)
    m0 = x[rng.choice(n, k, replace=False)].astype(np.float32).copy()
    v0 = rng.uniform(0.5, 2.0, size=(k, d)).astype(np.float32)
    return w0, m0, v0


@pytest.mark.parametrize("n,d,k,seed", [(3001, 200, 40, 11),     # padded 256
                                         (1500, 300, 70, 12),     # padded 384
                                         (4500, 500, 33, 13),     # padded 512, two chunks
                                         (2100, 513, 20, 14),     # padded 640
                                         (5000, 768, 24, 15)])    # padded 768, two chunks
def test_wide_ragged_per_step(ops, n, d, k, seed):
    x, _, _ = dg.custom(n, d, k, seed=seed)
    w0, m0, v0 = _init(x, k, seed)
    worst = _per_step(ops, x, w0, m0, v0, 3, label=f"wide n={n} d={d} k={k}")
    print(f"wide n={n} d={d} k={k} worst", worst)


def test_wide_loglik_rows_and_topm(ops):
    x, _, _ = dg.custom(6000, 256, 50, seed=21)
    w0, m0, v0 = _init(x, 50, 21)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0)
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt, w, mu, var = _to_dev(x, *th)
    tot, rows = ops.loglik(xt, w, mu, var, per_row=True)
    torch.cuda.synchronize()
    rL, rrows = oracle.loglik(x, *th, per_row=True)
    assert rel(tot.item(), rL) <= 1e-5
    g = rows.cpu().numpy()
    assert np.max(np.abs(g - rrows) / np.maximum(np.abs(rrows), 1.0)) <= 1e-6
    for m in (2, 3):
        idx, resp = ops.assign_topm(xt, w, mu, var, m)
        torch.cuda.synchronize()
        ridx, rresp, gap = oracle.topm(x, *th, m)
        ell_top = np.abs(np.log(np.maximum(rresp[:, 0], 1e-300)))
        _check_topm(idx.cpu().numpy(), resp.cpu().numpy(), ridx, rresp, gap, ell_top)


def test_wide_bf16_per_step(ops):
    x, _, _ = dg.custom(3000, 300, 40, seed=31, dtype="bf16")
    xf = dg.as_f32(x)
    w0, m0, v0 = _init(xf, 40, 31)
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    w, mu, var = _to_dev(w0, m0, v0)
    ws = ops.workspace(300, 40, DEV)
    for t in range(2):
        th = _host(w, mu, var)
        Lg = _gpu_step(ops, xt, w, mu, var, 1e-6, ws)
        rw, rmu, rv, rL, nk = oracle.em_step(xf, *th, 1e-6)
        assert rel(Lg, rL) <= 1e-5
        assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(xf), 5e-3, f"wide bf16 step {t}")


def test_wide_bitwise_determinism(ops):
    x, _, _ = dg.custom(5000, 400, 30, seed=41)
    w0, m0, v0 = _init(x, 30, 41)
    outs = []
    for _ in range(2):
        xt, w, mu, var = _to_dev(x, w0, m0, v0)
        L = _gpu_step(ops, xt, w, mu, var)
        outs.append((L, *_host(w, mu, var)))
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1:], outs[1][1:]):
        assert np.array_equal(a, b)


def test_wide_workload_prefix_step_and_top2(ops):
    # the wide many-component workload (D=768, K=16384) on a 20,000-row
    # prefix: one EM step per-step against the oracle, then the top-2 soft
    # assignment (IVF border-vector multi-assignment) on sampled rows
    W = dg.WORKLOADS["wide"]
    x = dg.rows(W, 20_000)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, 1, W.var_floor, label="wide workload prefix")
    print("wide workload prefix worst", worst)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0, W.var_floor)
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt, w, mu, var = _to_dev(x, *th)
    idx, resp = ops.assign_topm(xt, w, mu, var, 2)
    torch.cuda.synchronize()
    pick = np.random.default_rng(5).choice(len(x), 400, replace=False)
    ridx, rresp, gap = oracle.topm(x[pick], *th, 2)
    ell_top = np.abs(np.log(np.maximum(rresp[:, 0], 1e-300)))
    _check_topm(idx.cpu().numpy()[pick], resp.cpu().numpy()[pick], ridx, rresp, gap, ell_top)
