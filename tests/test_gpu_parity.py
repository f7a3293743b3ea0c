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


def _dev_x(x):
    """Rows on the device: fp32 as they are, bf16 bit patterns (uint16) as bf16."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _gpu_step(ops, xt, w, mu, var, floor=1e-6, ws=None):
    L = ops.em_step(xt, w, mu, var, floor, ws=ws)
    torch.cuda.synchronize()
    return L.item()


def _per_step(ops, x, w0, m0, v0, steps, floor=1e-6, tol=1e-4, ltol=1e-5, label="", path=None,
              first_path=None):
    xt = _dev_x(x)
    w, mu, var = _to_dev(w0, m0, v0)
    ws = ops.workspace(x.shape[1], len(w0), DEV)
    worst = {}
    for t in range(steps):
        th = _host(w, mu, var)
        Lg = _gpu_step(ops, xt, w, mu, var, floor, ws)
        rw, rmu, rv, rL, nk = oracle.em_step(x, *th, floor)
        assert rel(Lg, rL) <= ltol, f"{label} step {t}: loglik {Lg} vs {rL}"
        e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), tol, f"{label} step {t}")
        for kk in ("mu", "var", "w", "tiny_worst"):
            worst[kk] = max(worst.get(kk, 0.0), e[kk])
        # components with oracle mass in (0, 1), and those the GPU kills
        # while the oracle keeps them (asserted zero above)
        print(f"{label} step {t}: tiny components {e['n_tiny']}, killed {e['killed']}, "
              f"dead {e['n_dead']}")
        want = first_path if (t == 0 and first_path is not None) else path
        if want is not None:
            got = ops.estep_arithmetic(ws, DEV)
            allowed = (want,) if isinstance(want, int) else tuple(want)
            assert got in allowed, f"{label} step {t}: E-step arithmetic {got}, expected {allowed}"
            print(f"{label} step {t}: E-step arithmetic {got}")
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


@pytest.mark.parametrize("n,d,k,m,seed", [(3001, 20, 70, 1, 61), (64 * 7 + 5, 33, 17, 2, 62),
                                           (5000, 96, 200, 3, 63), (2500, 128, 40, 4, 64),
                                           (700, 5, 9, 4, 65)])
def test_assign_topm_int8(ops, n, d, k, m, seed):
    # integer-valued fp32 rows: the top-m pass runs on exact int8 slices
    # (32 rows per wave, top-2 or top-4 lists); ragged N, D, K and every m
    x = _int_data(n, d, k, seed, hi=120.0)
    w0, m0, v0 = _seed_params(x, k, seed)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0)
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt, w, mu, var = _to_dev(x, *th)
    ws = ops.workspace(d, k, DEV)
    idx, resp = ops.assign_topm(xt, w, mu, var, m, ws=ws)
    torch.cuda.synchronize()
    assert ops.estep_arithmetic(ws, DEV) == ops.GMM_ESTEP_INT8_SLICES
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
    worst = _per_step(ops, x, w0, m0, v0, 4, W.var_floor, label="descriptor prefix",
                      path=ops.GMM_ESTEP_INT8_SLICES_MSTEP)
    print("descriptor per-step worst", worst)


def test_tiny_mass_below_fp32_range_is_kept(ops):
    # Every row has l_1 - l_0 = -200 (rows at 0, unit-variance components at 0
    # and 20): r_1 ~ 1.4e-87 underflows in fp32 but not in fp64, so the
    # component keeps a nonzero mass and weight, as in the oracle.
    n = 1000
    x = np.zeros((n, 1), dtype=np.float32)
    w0 = np.array([0.5, 0.5], np.float32)
    m0 = np.array([[0.0], [20.0]], np.float32)
    v0 = np.ones((2, 1), np.float32)
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    _gpu_step(ops, xt, w, mu, var)
    rw, rmu, rv, rL, nk = oracle.em_step(x, w0, m0, v0)
    gw = w.cpu().numpy()
    # the weight N_1 / N is below fp32's range: stored as the smallest
    # positive fp32 value, so the component stays alive
    assert 0.0 < nk[1] < 1e-80 and gw[1] == np.nextafter(np.float32(0), np.float32(1))
    e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, n, 1e-4, "tiny mass")
    assert e["n_tiny"] == 1 and e["killed"] == 0


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


def test_descriptor_full_dense_step_matches_oracle(ops, descriptor_full):
    # The kernel bench.py times on every step after the first: two GPU steps
    # move away from the initial parameters (after which a row has tens of
    # nonzero responsibilities), then the third step on all 10^7 rows, three
    # 2^22-row chunks, is compared element by element with the oracle's step
    # from the same (GPU) parameters.
    W, x, w0, m0, v0 = descriptor_full
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    ws = ops.workspace(W.d, W.k, DEV)
    for _ in range(2):
        ops.em_step(xt, w, mu, var, W.var_floor, ws=ws)
    th = _host(w, mu, var)
    Lg = _gpu_step(ops, xt, w, mu, var, W.var_floor, ws)
    rw, rmu, rv, rL, nk = oracle.em_step(x, *th, W.var_floor)
    assert rel(Lg, rL) <= 1e-5
    e = assert_params_close(_host(w, mu, var), (rw, rmu, rv), nk, len(x), 1e-4,
                            "descriptor full dense step")
    print("descriptor full-size dense step:", e, "loglik rel", rel(Lg, rL))
    assert ops.device_status(ws, DEV) == ops.GMM_OK


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
    # bf16 data: the 5e-3 bar applies; the contractions run on split bf16
    W = dg.WORKLOADS["bf16_large"]
    x = dg.rows(W, 60_000)
    w0, m0, v0 = dg.init_params(W, x)
    worst = _per_step(ops, x, w0, m0, v0, 3, floor=W.var_floor, tol=5e-3, label="bf16_large prefix",
                      path=ops.GMM_ESTEP_BF16_SPLIT)
    print("bf16_large prefix per-step worst", worst)


# ---------------------------------------------------------------------------
# The E-step on exact int8 slices. Integer-valued data (features exact in a
# few 7-bit digits) selects it; real-valued fp32 data whose truncation cannot
# be bounded below 2^-20 nats keeps the fp64 E-step.
# ---------------------------------------------------------------------------
def _int_data(n, d, k, seed, scale=8.0, offset=40.0, hi=None):
    x, _, _ = dg.custom(n, d, k, seed=seed)
    x = np.clip(np.rint(x * scale + offset), 0, hi)
    return x.astype(np.float32)


def _seed_params(x, k, seed):
    rng = np.random.default_rng(seed)
    n, d = x.shape
    w0 = np.full(k, 1.0 / k, np.float32)
    m0 = x[rng.choice(n, k, replace=False)].copy()
    v0 = np.ones((k, d), np.float32)
    return w0, m0, v0


def test_estep_arithmetic_selection(ops):
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 20_000)
    w0, m0, v0 = dg.init_params(W, x)
    xt, w, mu, var = _to_dev(x, w0, m0, v0)
    ws = ops.workspace(W.d, W.k, DEV)
    ops.em_step(xt, w, mu, var, W.var_floor, ws=ws)
    assert ops.estep_arithmetic(ws, DEV) == ops.GMM_ESTEP_INT8_SLICES_MSTEP
    ops.loglik(xt, w, mu, var, ws=ws)
    assert ops.estep_arithmetic(ws, DEV) != ops.GMM_ESTEP_FP64
    T = dg.WORKLOADS["tiny"]
    xr = dg.rows(T)
    xt2, w2, mu2, var2 = _to_dev(xr, *dg.init_params(T, xr))
    ws2 = ops.workspace(T.d, T.k, DEV)
    ops.em_step(xt2, w2, mu2, var2, T.var_floor, ws=ws2)
    assert ops.estep_arithmetic(ws2, DEV) == ops.GMM_ESTEP_FP64


@pytest.mark.parametrize("n,d,k,seed", [(1007, 5, 3, 1), (3001, 20, 70, 2), (64 * 7 + 5, 33, 17, 4),
                                         (5000, 128, 100, 5), (3000, 96, 1024, 6), (700, 1, 9, 7)])
def test_int8_path_ragged_integer_data(ops, n, d, k, seed):
    # values in [0, 120]: |a| <= 127, one digit for a and two for a^2 (at
    # d = 128 a wider range needs more chunks than the int8 kernels hold,
    # and the fp64 E-step runs instead)
    x = _int_data(n, d, k, seed, hi=120.0)
    w0, m0, v0 = _seed_params(x, k, seed)
    worst = _per_step(ops, x, w0, m0, v0, 3, label=f"int8 n={n} d={d} k={k}",
                      path=ops.GMM_ESTEP_INT8_SLICES if d > 112 else ops.GMM_ESTEP_INT8_SLICES_MSTEP)
    print(f"int8 path n={n} d={d} k={k} per-step worst", worst)


@pytest.mark.parametrize("hi,scale,step", [(1000.0, 60.0, 1.0), (120.0, 8.0, 0.5), (60.0, 4.0, 0.25)])
def test_int8_path_multi_digit_features(ops, hi, scale, step):
    # |a| beyond 127 needs two digits for a and three for a^2; values on a
    # grid of 1/2 or 1/4 need one more low digit each: every case is still
    # exact in at most three digits per column, so the int8 path runs
    x, _, _ = dg.custom(3000, 32, 40, seed=8)
    x = (np.clip(np.rint((x * scale + hi / 2) / step), 0, hi / step) * step).astype(np.float32)
    w0, m0, v0 = _seed_params(x, 40, 8)
    # (a tile whose coefficients need more digit levels than the statistics
    # pass holds in registers runs the fp64 statistics pass)
    _per_step(ops, x, w0, m0, v0, 3, label=f"int8 range {hi} grid {step}",
              path=(ops.GMM_ESTEP_INT8_SLICES, ops.GMM_ESTEP_INT8_SLICES_MSTEP))


def test_int8_mstep_single_digit_squares(ops):
    # integers in [0, 16]: |a| <= 8 after the shift, so a and a^2 are each
    # one exact digit (the (1, 1) variant of the int8 M-step)
    rng = np.random.default_rng(23)
    n, d, k = 4000 + 11, 24, 40
    x = rng.integers(0, 17, size=(n, d)).astype(np.float32)
    w0, m0, v0 = _seed_params(x, k, 23)
    _per_step(ops, x, w0, m0, v0, 3, label="int8 one-digit squares",
              path=ops.GMM_ESTEP_INT8_SLICES_MSTEP)


def test_int8_estep_with_fp64_mstep(ops):
    # data on a grid of 2^-12: a is exact in three digits, a^2 is not, so the
    # M-step stays fp64; variances so large that the truncation of a^2 moves a
    # log-density by far less than 2^-20 nats, so the E-step runs on int8
    # slices (the int8 E-step with the fp64 M-step, one step)
    rng = np.random.default_rng(21)
    n, d, k = 3000 + 37, 16, 24
    x = (np.rint(rng.uniform(0.0, 120.0, size=(n, d)) * 4096.0) / 4096.0).astype(np.float32)
    w0 = np.full(k, 1.0 / k, np.float32)
    m0 = x[rng.choice(n, k, replace=False)].copy()
    v0 = np.full((k, d), 1.0e7, np.float32)
    _per_step(ops, x, w0, m0, v0, 1, label="int8 E-step, fp64 M-step",
              path=ops.GMM_ESTEP_INT8_SLICES_BOTH)


def test_int8_path_rows_beyond_one_chunk(ops):
    n = (1 << 22) + 1234
    x = _int_data(n, 8, 4, 9)
    w0, m0, v0 = _seed_params(x, 4, 9)
    _per_step(ops, x, w0, m0, v0, 1, label="int8 two chunks", path=ops.GMM_ESTEP_INT8_SLICES_MSTEP)


def test_int8_loglik_rows(ops):
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 50_000)
    w0, m0, v0 = dg.init_params(W, x)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0, W.var_floor)
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt, w, mu, var = _to_dev(x, *th)
    ws = ops.workspace(W.d, W.k, DEV)
    tot, rows = ops.loglik(xt, w, mu, var, per_row=True, ws=ws)
    assert ops.estep_arithmetic(ws, DEV) != ops.GMM_ESTEP_FP64
    rL, rrows = oracle.loglik(x, *th, per_row=True)
    assert rel(tot.item(), rL) <= 1e-9
    g = rows.cpu().numpy()
    assert np.max(np.abs(g - rrows) / np.maximum(np.abs(rrows), 1.0)) <= 1e-6


# ---------------------------------------------------------------------------
# The split-bf16 path for bf16 data: features [a^2 hi, a^2 lo, a] exact in
# bf16, coefficients and responsibilities split in bf16 parts, fp32 slices
# added in fp64. bf16 data is held to the 5e-3 bar; the log-likelihood to
# 1e-5 relative.
# ---------------------------------------------------------------------------
def _bf16_data(n, d, k, seed, scale=0.25):
    # planted mixture scaled so that the shift is 0 and a = x stays a bf16
    # value: means ~ N(0, (4 scale)^2), sd in [scale/2, 2 scale]
    x, _, _ = dg.custom(n, d, k, seed=seed, spread=4.0 * scale, sd_lo=0.5 * scale, sd_hi=2.0 * scale)
    return dg.f64_to_bf16_bits(x.astype(np.float64))


def _bf16_seed_params(x, k, seed):
    rng = np.random.default_rng(seed)
    n, d = x.shape
    w0 = np.full(k, 1.0 / k, np.float32)
    m0 = dg.bf16_bits_to_f32(x[rng.choice(n, k, replace=False)]).copy()
    v0 = np.ones((k, d), np.float32)
    return w0, m0, v0


@pytest.mark.parametrize("n,d,k,seed", [(1007, 5, 3, 31), (3001, 20, 70, 32), (64 * 7 + 5, 33, 17, 33),
                                         (2500, 64, 130, 34), (4000, 100, 48, 35), (3000, 128, 257, 36),
                                         (700, 1, 9, 37)])
def test_bf16_split_ragged_shapes(ops, n, d, k, seed):
    # every slice count (d up to 32, 64, 96, 128), ragged rows, components
    # and dimensions; four steps from seeded rows. The first step (unit
    # variances) runs on split bf16; later ones may fall back to fp64 when a
    # component narrows onto a few rows and the rounding estimate exceeds
    # its bound.
    x = _bf16_data(n, d, k, seed)
    w0, m0, v0 = _bf16_seed_params(x, k, seed)
    worst = _per_step(ops, x, w0, m0, v0, 4, tol=5e-3, label=f"bf16 split n={n} d={d} k={k}",
                      first_path=ops.GMM_ESTEP_BF16_SPLIT,
                      path=(ops.GMM_ESTEP_BF16_SPLIT, ops.GMM_ESTEP_FP64))
    print(f"bf16 split n={n} d={d} k={k} per-step worst", worst)
    # far below the bar in practice: means and weights keep about fp32
    # accuracy; a variance carries the fp32 rounding of its tile sums times
    # E[x^2] / var (no shift on this path: 1.5e-4 for a two-row component
    # at mean -1.4 and variance 1.4e-4, as a CPU emulation of the same
    # arithmetic also gives)
    assert worst["mu"] < 1e-4 and worst["w"] < 1e-4 and worst["var"] < 1e-3


def test_bf16_split_falls_back_to_fp64(ops):
    # (1) a value whose square's low bits fall below bf16's normal range
    # (1e-20 ~ 2^-66); (2) components so narrow that the fp32 rounding
    # estimate exceeds the accepted bound: both run the fp64 contractions
    rng = np.random.default_rng(41)
    n, d, k = 2000 + 3, 16, 12
    x1 = _bf16_data(n, d, k, 41)
    x1[5, 3] = dg.f64_to_bf16_bits(np.array([1e-20]))[0]
    w0, m0, v0 = _bf16_seed_params(x1, k, 41)
    _per_step(ops, x1, w0, m0, v0, 1, tol=5e-3, label="bf16 tiny value", path=ops.GMM_ESTEP_FP64)
    x2 = _bf16_data(n, d, k, 42, scale=1.0)
    w0, m0, _ = _bf16_seed_params(x2, k, 42)
    v0 = np.full((k, d), 1e-4, np.float32)
    _per_step(ops, x2, w0, m0, v0, 1, tol=5e-3, label="bf16 narrow", path=ops.GMM_ESTEP_FP64)
    # integer-valued bf16 data takes the exact int8 path instead
    x3 = dg.f64_to_bf16_bits(np.rint(rng.uniform(0, 100, size=(n, d))))
    w0, m0, v0 = _bf16_seed_params(x3, k, 43)
    _per_step(ops, x3, w0, m0, v0, 1, tol=5e-3, label="bf16 integers",
              path=ops.GMM_ESTEP_INT8_SLICES_MSTEP)


def test_bf16_split_loglik_rows_and_determinism(ops):
    W = dg.WORKLOADS["bf16_large"]
    x = dg.rows(W, 30_000)
    w0, m0, v0 = dg.init_params(W, x)
    rw, rmu, rv, *_ = oracle.em_step(x, w0, m0, v0, W.var_floor)
    th = [a.astype(np.float32) for a in (rw, rmu, rv)]
    xt = _dev_x(x)
    w, mu, var = _to_dev(*th)
    ws = ops.workspace(W.d, W.k, DEV)
    tot, rows = ops.loglik(xt, w, mu, var, per_row=True, ws=ws)
    assert ops.estep_arithmetic(ws, DEV) == ops.GMM_ESTEP_BF16_SPLIT
    g = rows.cpu().numpy()
    rL, rrows = oracle.loglik(x, *th, per_row=True)
    err = np.abs(g - rrows)
    print("bf16 split per-row loglik: max abs err", err.max(), "rel total", rel(tot.item(), rL))
    # rows are sums of 128 dims of terms up to a few hundred nats: the fp32
    # slices keep them within 1e-3 nats
    assert err.max() < 1e-3
    assert rel(tot.item(), rL) <= 1e-6
    # two identical steps give identical bits
    outs = []
    for _ in range(2):
        w2, mu2, var2 = _to_dev(*th)
        L = ops.em_step(xt, w2, mu2, var2, W.var_floor, ws=ws)
        torch.cuda.synchronize()
        outs.append([L.item()] + [a.copy() for a in _host(w2, mu2, var2)])
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1:], outs[1][1:]):
        assert np.array_equal(a, b)


def test_bf16_split_rows_beyond_one_chunk(ops):
    # two 2^22-row chunks with a ragged tail, the launch configuration of the
    # full-size workload (chunked normaliser and statistics passes)
    n = (1 << 22) + 3 * 4096 + 77
    x = _bf16_data(n, 24, 6, 51)
    w0, m0, v0 = _bf16_seed_params(x, 6, 51)
    _per_step(ops, x, w0, m0, v0, 2, tol=5e-3, label="bf16 split two chunks",
              path=ops.GMM_ESTEP_BF16_SPLIT)
