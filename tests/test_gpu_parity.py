"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Every case uses the same seeded inputs on both sides. Per-step comparisons
feed the GPU's fp32 parameters (converted exactly) to the oracle, so they
measure one step's kernel error; end-to-end comparisons run both sides from
the same initial parameters.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gmm_em_amd import datagen as dg  # noqa: E402
from oracle import oracle  # noqa: E402
from tests.parity import assert_params_close, param_errors, rel  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    from gmm_em_amd import ops as o

    return o


def _to_dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def _host(*ts):
    return [t.detach().cpu().numpy() for t in ts]


def _gpu_step(ops, xt, w, mu, var, floor=1e-6, ws=None):
    L = ops.em_step(xt, w, mu, var, floor, ws=ws)
    torch.cuda.synchronize()
    return L.item()


def _per_step(ops, x, w0, m0, v0, steps, floor=1e-6, tol=1e-4, ltol=1e-5, label=""):
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    ws = ops.workspace(x.shape[1], len(w0), DEV)
    worst = {}
    for t in range(steps):
        th = _host(w, mu, var)
        Lg = _gpu_step(ops, xt, w, mu, var, floor, ws)
        rw, rmu, rv, rL, nk = oracle.em_step(x, *th, floor)
        assert rel(Lg, rL) <= ltol, f"{label} step {t}: loglik {Lg} vs {rL}"
        e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), tol, f"{label} step {t}")
        for kk in ("mu", "var", "w"):
            worst[kk] = max(worst.get(kk, 0.0), e[kk])
    assert ops.device_status(ws, DEV) == ops.GMM_OK
    return worst


def test_tiny_per_step_20_iterations(ops):
    W = dg.WORKLOADS["tiny"]
    x = dg.rows(W)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, W.iters, W.var_floor, label="tiny")
    print("tiny per-step worst", worst)


def test_tiny_end_to_end_fit(ops):
    W = dg.WORKLOADS["tiny"]
    x = dg.rows(W)
    w0, m0, v0 = dg.init_params(W, x)
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    hist, done = ops.fit(xt, w, mu, var, W.var_floor, W.iters)
    torch.cuda.synchronize()
    assert done == W.iters
    rw, rmu, rv, rhist = oracle.fit(x, w0, m0, v0, W.var_floor, W.iters)
    h = hist.cpu().numpy()
    assert np.all(np.abs(h - rhist) / np.abs(rhist) <= 1e-5), (h, rhist)
    nk = rw * len(x)
    e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), 1e-4, "tiny fit")
    print("tiny end-to-end", e)
    assert np.all(np.diff(h) >= -1e-6 * np.abs(h[1:]))  # monotone within fp32 noise


@pytest.mark.parametrize("n,d,k,seed", [(1007, 5, 3, 1), (3001, 20, 70, 2), (130, 16, 64, 3),
                                         (64 * 7 + 5, 33, 17, 4), (5000, 128, 100, 5)])
def test_ragged_shapes(ops, n, d, k, seed):
    x, pl, _ = dg.custom(n, d, k, seed=seed)
    rng = np.random.default_rng(seed)
    w0 = rng.dirichlet(np.ones(k)).astype(np.float32)
    m0 = x[rng.choice(n, k, replace=False)].copy()
    v0 = rng.uniform(0.5, 2.0, size=(k, d)).astype(np.float32)
    _per_step(ops, x, w0, m0, v0, 3, label=f"ragged n={n} d={d} k={k}")


def test_single_component_closed_form(ops):
    rng = np.random.default_rng(7)
    x = (rng.normal(3.0, 2.0, size=(20000, 12))).astype(np.float32)
    xt, w, mu, var = _to_dev(x, np.ones(1, np.float32), np.zeros((1, 12), np.float32),
                             np.ones((1, 12), np.float32))
    _gpu_step(ops, xt, w, mu, var)
    X = x.astype(np.float64)
    gw, gmu, gv = _host(w, mu, var)
    assert gw[0] == 1.0
    np.testing.assert_allclose(gmu[0], X.mean(0), rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(gv[0], X.var(0), rtol=1e-4)


def test_loglik_total_and_rows(ops):
    W = dg.WORKLOADS["embed"]
    x = dg.rows(W, 50_000)
    w0, m0, v0 = dg.init_params(W, x)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0)  # a fitted-ish parameter set
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt, w, mu, var = _to_dev(x, *th)
    tot, rows = ops.loglik(xt, w, mu, var, per_row=True)
    torch.cuda.synchronize()
    rL, rrows = oracle.loglik(x, *th, per_row=True)
    assert rel(tot.item(), rL) <= 1e-5
    g = rows.cpu().numpy().astype(np.float64)
    # the per-row normaliser is m + log(s) with m in fp64 and s an fp32 sum
    assert np.max(np.abs(g - rrows) / np.maximum(np.abs(rrows), 1.0)) <= 1e-6


def test_loglik_empty_input(ops):
    xt = torch.zeros((0, 8), dtype=torch.float32, device=DEV)
    w, mu, var = _to_dev(np.full(4, 0.25, np.float32), np.zeros((4, 8), np.float32),
                         np.ones((4, 8), np.float32))
    tot = ops.loglik(xt, w, mu, var)
    torch.cuda.synchronize()
    assert tot.item() == 0.0


def _check_topm(idx, resp, ridx, rresp, gap, ell_scale):
    same = np.all(idx == ridx, axis=1)
    # a different choice is only allowed where the oracle's own margin is tiny
    near_tie = gap < 1e-3 * np.maximum(1.0, ell_scale)
    assert np.all(same | near_tie), f"{np.sum(~same & ~near_tie)} rows differ"
    ok = same
    np.testing.assert_allclose(resp[ok], rresp[ok], rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("wl,n,m", [("tiny", 10_000, 2), ("embed", 20_000, 2), ("tiny", 3001, 3)])
def test_assign_topm(ops, wl, n, m):
    W = dg.WORKLOADS[wl]
    x = dg.rows(W, n)
    w0, m0, v0 = dg.init_params(W, x)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0)
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt, w, mu, var = _to_dev(x, *th)
    idx, resp = ops.assign_topm(xt, w, mu, var, m)
    torch.cuda.synchronize()
    ridx, rresp, gap = oracle.topm(x, *th, m)
    ell_top = np.abs(np.log(np.maximum(rresp[:, 0], 1e-300)))
    _check_topm(idx.cpu().numpy(), resp.cpu().numpy(), ridx, rresp, gap, ell_top)


def test_embed_prefix_per_step(ops):
    W = dg.WORKLOADS["embed"]
    x = dg.rows(W, 100_000)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, 3, label="embed prefix")
    print("embed per-step worst", worst)


def test_embed_full_per_step(ops):
    # the embedding-like workload at its full size (N = 1,000,000, D = 128,
    # K = 256), three EM steps from the seeded initial parameters
    W = dg.WORKLOADS["embed"]
    x = dg.rows(W)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, 3, W.var_floor, label="embed full")
    print("embed full-size per-step worst", worst)


def test_descriptor_prefix_per_step(ops):
    # integer descriptor data: after one step some components sit at the
    # variance floor in some dims (w = 1e6), the hardest case for the
    # expanded Gaussian exponent
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 200_000)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, 4, W.var_floor, label="descriptor prefix")
    print("descriptor per-step worst", worst)


def test_bitwise_determinism(ops):
    W = dg.WORKLOADS["embed"]
    x = dg.rows(W, 30_000)
    w0, m0, v0 = dg.init_params(W, x)
    outs = []
    for _ in range(2):
        xt, w, mu, var = _to_dev(x, w0, m0, v0)
        L = _gpu_step(ops, xt, w, mu, var)
        outs.append((L, *_host(w, mu, var)))
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1:], outs[1][1:]):
        assert np.array_equal(a, b)


def test_invalid_parameters_reported(ops):
    x = np.random.default_rng(3).normal(size=(500, 4)).astype(np.float32)
    v0 = np.ones((2, 4), np.float32)
    v0[1, 2] = 0.0
    xt, w, mu, var = _to_dev(x, np.array([0.5, 0.5], np.float32), x[:2].copy(), v0)
    ws = ops.workspace(4, 2, DEV)
    ops.em_step(xt, w, mu, var, ws=ws)
    assert ops.device_status(ws, DEV) == ops.GMM_E_PARAMS
    assert np.all(np.isnan(w.cpu().numpy()))
    # a valid call on the same workspace clears the status
    xt, w, mu, var = _to_dev(x, np.array([0.5, 0.5], np.float32), x[:2].copy(), np.ones((2, 4), np.float32))
    ops.em_step(xt, w, mu, var, ws=ws)
    assert ops.device_status(ws, DEV) == ops.GMM_OK


def test_rows_beyond_one_chunk(ops):
    # more rows than one 2^22-row chunk: normalisers and partials carry over
    n = (1 << 22) + 1234
    x, pl, _ = dg.custom(n, 8, 4, seed=9)
    rng = np.random.default_rng(9)
    w0 = np.full(4, 0.25, np.float32)
    m0 = x[rng.choice(n, 4, replace=False)].copy()
    v0 = np.ones((4, 8), np.float32)
    _per_step(ops, x, w0, m0, v0, 1, label="two chunks")


def test_bf16_input(ops):
    x, pl, _ = dg.custom(20_000, 32, 12, seed=11, dtype="bf16")
    rng = np.random.default_rng(11)
    w0 = np.full(12, 1 / 12, np.float32)
    m0 = dg.bf16_bits_to_f32(x[rng.choice(len(x), 12, replace=False)]).copy()
    v0 = np.ones((12, 32), np.float32)
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    w, mu, var = _to_dev(w0, m0, v0)
    Lg = _gpu_step(ops, xt, w, mu, var)
    rw, rmu, rv, rL, nk = oracle.em_step(x, w0, m0, v0)
    assert rel(Lg, rL) <= 1e-5
    assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), 5e-3, "bf16")


# ---------------------------------------------------------------------------
# Full-size checks on the headline workload, in the configuration bench.py
# times (N = 10,000,000 rows, D = 96, K = 1024, three 2^22-row chunks).
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def descriptor_full():
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W)
    w0, m0, v0 = dg.init_params(W, x)
    return W, x, w0, m0, v0


def test_descriptor_full_first_step_matches_oracle(ops, descriptor_full):
    W, x, w0, m0, v0 = descriptor_full
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    Lg = _gpu_step(ops, xt, w, mu, var, W.var_floor)
    rw, rmu, rv, rL, nk = oracle.em_step(x, w0, m0, v0, W.var_floor)
    assert rel(Lg, rL) <= 1e-5
    e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), 1e-4, "descriptor full step 0")
    print("descriptor full-size step 0:", e, "loglik rel", rel(Lg, rL))
    assert abs(float(w.sum().item()) - 1.0) < 1e-5


def test_descriptor_full_loglik_rows_and_topm_sampled(ops, descriptor_full):
    W, x, w0, m0, v0 = descriptor_full
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    ws = ops.workspace(W.d, W.k, DEV)
    for _ in range(2):  # move away from the initial parameters
        ops.em_step(xt, w, mu, var, W.var_floor, ws=ws)
    th = _host(w, mu, var)
    tot, rows = ops.loglik(xt, w, mu, var, per_row=True, ws=ws)
    idx, resp = ops.assign_topm(xt, w, mu, var, 2, ws=ws)
    torch.cuda.synchronize()
    g = rows.cpu().numpy()
    # the total is the fixed-order sum of the rows; the rows span all chunks
    assert rel(tot.item(), float(np.sum(g))) <= 1e-9
    rng = np.random.default_rng(123)
    pick = np.sort(rng.choice(len(x), 4000, replace=False))
    pick[-1] = len(x) - 1  # the ragged tail of the last chunk
    rL, rrows = oracle.loglik(x[pick], *th, per_row=True)
    np.testing.assert_allclose(g[pick], rrows, rtol=1e-6, atol=1e-6)
    ridx, rresp, gap = oracle.topm(x[pick], *th, 2)
    ell_top = np.abs(np.log(np.maximum(rresp[:, 0], 1e-300)))
    _check_topm(idx.cpu().numpy()[pick], resp.cpu().numpy()[pick], ridx, rresp, gap, ell_top)


def test_bf16_large_prefix_per_step(ops):
    W = dg.WORKLOADS["bf16_large"]
    x = dg.rows(W, 60_000)
    w0, m0, v0 = dg.init_params(W, x)
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    w, mu, var = _to_dev(w0, m0, v0)
    ws = ops.workspace(W.d, W.k, DEV)
    for t in range(2):
        th = _host(w, mu, var)
        Lg = _gpu_step(ops, xt, w, mu, var, W.var_floor, ws)
        rw, rmu, rv, rL, nk = oracle.em_step(x, *th, W.var_floor)
        assert rel(Lg, rL) <= 1e-5
        # bf16 data: the 5e-3 bar applies; the arithmetic itself is fp64
        e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), 5e-3, f"bf16_large step {t}")
        print(f"bf16_large prefix step {t}:", e)


# ---------------------------------------------------------------------------
# Both schedules of the EM step (the default two-pass schedule and the
# opt-in cooperative single pass) against the oracle.
# ---------------------------------------------------------------------------
@pytest.fixture(params=["two_pass", "coop"])
def schedule(request, monkeypatch):
    monkeypatch.setenv("GMM_EM_SCHEDULE", request.param)
    return request.param


def test_schedules_descriptor_prefix(ops, schedule):
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 150_000)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, 3, W.var_floor, label=f"descriptor {schedule}")
    print(schedule, "descriptor per-step worst", worst)


@pytest.mark.parametrize("n,d,k,seed", [(1007, 5, 3, 1), (3001, 20, 70, 2), (5000, 128, 100, 5)])
def test_schedules_ragged(ops, schedule, n, d, k, seed):
    x, pl, _ = dg.custom(n, d, k, seed=seed)
    rng = np.random.default_rng(seed)
    w0 = rng.dirichlet(np.ones(k)).astype(np.float32)
    m0 = x[rng.choice(n, k, replace=False)].copy()
    v0 = rng.uniform(0.5, 2.0, size=(k, d)).astype(np.float32)
    _per_step(ops, x, w0, m0, v0, 2, label=f"{schedule} n={n} d={d} k={k}")


def test_schedules_agree_and_are_deterministic(ops, monkeypatch):
    W = dg.WORKLOADS["embed"]
    x = dg.rows(W, 40_000)
    w0, m0, v0 = dg.init_params(W, x)
    res = {}
    for sch in ("coop", "coop", "two_pass"):
        monkeypatch.setenv("GMM_EM_SCHEDULE", sch)
        xt, w, mu, var = _to_dev(x, w0, m0, v0)
        ws = ops.workspace(W.d, W.k, DEV)
        L = ops.em_step(xt, w, mu, var, ws=ws)
        assert ops.device_status(ws, DEV) == ops.GMM_OK
        out = (L.item(), *_host(w, mu, var))
        if sch in res:  # bitwise repeatable
            assert out[0] == res[sch][0]
            for a, b in zip(out[1:], res[sch][1:]):
                assert np.array_equal(a, b)
        res[sch] = out
    # the two schedules merge the per-row partial sums in different orders:
    # equal to rounding
    assert rel(res["coop"][0], res["two_pass"][0]) <= 1e-10
    np.testing.assert_allclose(res["coop"][2], res["two_pass"][2], rtol=1e-6, atol=1e-7)
