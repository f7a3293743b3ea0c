"""The allocation-free EM step (gmm_em_step_noalloc) against gmm_em_step.

Both are called through the C ABI on the same seeded inputs and parameters;
the allocation-free one uses the library's device scratch instead of a
workspace. Two calls in a row, the second on a smaller input (the scratch
keeps the first call's contents), each compared with the workspace entry
point to the parity bar: parameters within 1e-6 relative (the two plans
differ only in reduction order), log-likelihood within 1e-12. A shape whose
workspace cannot fit the scratch is refused with GMM_E_UNSUPPORTED.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gmm_em_amd import datagen as dg  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ops():
    from gmm_em_amd import ops as o

    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    o.lib.gmm_em_step_noalloc.argtypes = [vp, i64, i32, i64, i32, vp, vp, vp, i32, f32, vp, vp]
    o.lib.gmm_em_step_noalloc.restype = ctypes.c_int
    return o


def _noalloc(ops, xt, w, mu, var, floor):
    L = torch.empty((), dtype=torch.float64, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dt = ops.GMM_BF16 if xt.dtype == torch.bfloat16 else ops.GMM_F32
    rc = ops.lib.gmm_em_step_noalloc(p(xt), xt.shape[0], xt.shape[1], xt.shape[1], dt, p(w), p(mu),
                                     p(var), w.shape[0], floor, p(L),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, L


def _compare(ops, x, w0, m0, v0, floor, label, path=None):
    print(f"# {label}: N={x.shape[0]} D={x.shape[1]} K={len(w0)}", flush=True)
    if x.dtype == np.uint16:  # bf16 bit patterns
        xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x).to(DEV)
    ref = [torch.from_numpy(a).to(DEV) for a in (w0, m0, v0)]
    got = [t.clone() for t in ref]
    ws = ops.workspace(x.shape[1], len(w0), DEV)
    Lr = ops.em_step(xt, *ref, floor, ws=ws)
    if path is not None:
        assert ops.estep_arithmetic(ws, DEV) == path
    rc, Lg = _noalloc(ops, xt, *got, floor)
    torch.cuda.synchronize()
    assert rc == ops.GMM_OK, rc
    assert abs(Lg.item() - Lr.item()) <= 1e-12 * abs(Lr.item()), (Lg.item(), Lr.item())
    for a, b in zip(got, ref):
        a, b = a.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-30)


def test_noalloc_matches_workspace_entry_point_twice(ops):
    W = dg.WORKLOADS["descriptor"]
    x = dg.rows(W, 300_000)
    _compare(ops, x, *dg.init_params(W, x), W.var_floor, "descriptor prefix")
    T = dg.WORKLOADS["tiny"]
    xs = dg.rows(T)
    _compare(ops, xs, *dg.init_params(T, xs), T.var_floor, "tiny (smaller, after the first)")


def test_noalloc_bf16_split_path(ops):
    # bf16 data on the split-bf16 path: the scratch also holds that path's
    # coefficient pieces; a larger call, then a smaller one
    B = dg.WORKLOADS["bf16_large"]
    xb = dg.rows(B, 120_000)
    _compare(ops, xb, *dg.init_params(B, xb), B.var_floor, "bf16_large prefix",
             path=ops.GMM_ESTEP_BF16_SPLIT)
    xs = xb[:5_003]
    _compare(ops, xs, *dg.init_params(B, xs), B.var_floor, "bf16_large smaller prefix",
             path=ops.GMM_ESTEP_BF16_SPLIT)


def test_noalloc_rejects_shapes_beyond_the_scratch(ops):
    d, k = 768, 16384
    xt = torch.zeros((64, d), dtype=torch.float32, device=DEV)
    w = torch.full((k,), 1.0 / k, dtype=torch.float32, device=DEV)
    mu = torch.zeros((k, d), dtype=torch.float32, device=DEV)
    var = torch.ones((k, d), dtype=torch.float32, device=DEV)
    rc, _ = _noalloc(ops, xt, w, mu, var, 1e-6)
    assert rc == ops.GMM_E_UNSUPPORTED
