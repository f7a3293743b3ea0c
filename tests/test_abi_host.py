"""Host-side checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gmm_em.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gmm_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def ops():
    from gmm_em_amd import ops as o

    return o


def test_library_exports_every_declared_symbol(ops):
    names = _declared()
    assert {"gmm_em_step", "gmm_fit", "gmm_loglik", "gmm_assign_topm", "gmm_kmeans_step",
            "gmm_ivf_build"} <= set(names)
    for nm in names:
        assert hasattr(ops.lib, nm), nm
    assert ops.lib.gmm_version() >= 100


def test_workspace_size_rules(ops):
    a = ops.workspace_bytes(96, 1024)
    assert a > 0 and a % 256 == 0
    assert ops.workspace_bytes(96, 1024) == a  # no dependence on rows by construction
    assert ops.workspace_bytes(0, 8) == 0 and ops.workspace_bytes(16, 0) == 0
    assert ops.workspace_bytes(100000, 8) == 0  # unsupported dimension
    assert ops.workspace_bytes(96, 1025) >= a  # grows with K (never with the row count)


def test_status_strings(ops):
    for c in range(7):
        assert ops.lib.gmm_status_string(c).decode()
    assert ops.lib.gmm_status_string(99).decode() == "unknown status"


def _em(ops, **kw):
    a = dict(x=1, n=10, d=4, ldx=4, dt=0, w=1, mu=1, var=1, k=2, floor=1e-6, ll=None, ws=1, wsb=0,
             st=None)
    a.update(kw)
    return ops.lib.gmm_em_step(a["x"], a["n"], a["d"], a["ldx"], a["dt"], a["w"], a["mu"], a["var"],
                               a["k"], a["floor"], a["ll"], a["ws"], a["wsb"], a["st"])


def test_bad_arguments_rejected_before_any_launch(ops):
    # every case is decided on the host: no device pointer is dereferenced
    assert _em(ops, n=0) == ops.GMM_E_WORKSPACE or _em(ops, n=0) == ops.GMM_E_INVALID
    assert _em(ops, n=-1) == ops.GMM_E_INVALID
    assert _em(ops, d=0) == ops.GMM_E_INVALID
    assert _em(ops, ldx=3) == ops.GMM_E_INVALID
    assert _em(ops, k=0) == ops.GMM_E_INVALID
    assert _em(ops, x=None) == ops.GMM_E_INVALID
    assert _em(ops, mu=None) == ops.GMM_E_INVALID
    assert _em(ops, dt=7) == ops.GMM_E_DTYPE
    assert _em(ops, d=4000, ldx=4000) == ops.GMM_E_UNSUPPORTED
    assert _em(ops, ldx=1 << 24) == ops.GMM_E_UNSUPPORTED  # row stride past 32-bit tile offsets
    assert _em(ops, ws=None) == ops.GMM_E_WORKSPACE
    assert _em(ops, wsb=16) == ops.GMM_E_WORKSPACE
    need = ops.workspace_bytes(4, 2)
    assert _em(ops, ws=256 + 1, wsb=need) == ops.GMM_E_WORKSPACE  # misaligned
    # n == 0 and a bad floor are invalid for an EM step once the workspace is fine
    assert _em(ops, n=0, ws=256, wsb=need) == ops.GMM_E_INVALID
    assert _em(ops, floor=float("nan"), ws=256, wsb=need) == ops.GMM_E_INVALID
    assert _em(ops, floor=-1.0, ws=256, wsb=need) == ops.GMM_E_INVALID


def test_fit_and_topm_argument_checks(ops):
    f = ops.lib.gmm_fit
    need = ops.workspace_bytes(4, 2)
    assert f(1, 10, 4, 4, 0, 1, 1, 1, 2, 1e-6, -1, 0.0, None, None, 256, need, None) == ops.GMM_E_INVALID
    assert f(1, 10, 4, 4, 0, 1, 1, 1, 2, 1e-6, 3, -1.0, None, None, 256, need, None) == ops.GMM_E_INVALID
    t = ops.lib.gmm_assign_topm
    assert t(1, 10, 4, 4, 0, 1, 1, 1, 2, 0, 1, 1, 256, need, None) == ops.GMM_E_INVALID
    assert t(1, 10, 4, 4, 0, 1, 1, 1, 2, 3, 1, 1, 256, need, None) == ops.GMM_E_INVALID
    assert t(1, 10, 4, 4, 0, 1, 1, 1, 2, 1, None, 1, 256, need, None) == ops.GMM_E_INVALID


def test_kmeans_argument_checks(ops):
    # host-side rejections happen before any device call
    km = ops.lib.gmm_kmeans_step
    need = ops.workspace_bytes(4, 2)
    assert km(1, 0, 4, 4, 0, 1, 2, None, None, 256, need, None) == ops.GMM_E_INVALID  # n = 0
    assert km(1, 10, 4, 4, 0, None, 2, None, None, 256, need, None) == ops.GMM_E_INVALID
    assert km(1, 10, 4, 3, 0, 1, 2, None, None, 256, need, None) == ops.GMM_E_INVALID  # ldx < d
    assert km(1, 10, 4, 4, 7, 1, 2, None, None, 256, need, None) == ops.GMM_E_DTYPE
    assert km(1, 10, 4, 4, 0, 1, 2, None, None, 256, need - 1, None) == ops.GMM_E_WORKSPACE
    assert km(1, 10, 800, 800, 0, 1, 2, None, None, 256, need, None) == ops.GMM_E_UNSUPPORTED


def test_ivf_workspace_and_argument_checks(ops):
    wb = ops.lib.gmm_ivf_workspace_bytes
    assert wb(1000, 2, 64) > 0 and wb(1000, 2, 64) % 256 == 0
    assert wb(0, 2, 64) > 0                       # empty input still needs the counters
    assert wb(1000, 2, 16385) == 0                # more lists than LDS counters
    assert wb(1 << 30, 2, 64) == 0                # n*m beyond 32-bit positions
    assert wb(-1, 2, 64) == 0 and wb(10, 0, 64) == 0 and wb(10, 2, 0) == 0
    # the counters matrix stays bounded: tiles grow with n instead
    assert wb(50_000_000, 2, 4096) <= (1 << 26) + 4096 * 4 + 512
    b = ops.lib.gmm_ivf_build
    need = wb(100, 2, 8)
    assert b(1, 1, 100, 2, 8, 0.0, None, 1, None, 256, need, None) == ops.GMM_E_INVALID  # no offsets
    assert b(None, 1, 100, 2, 8, 0.0, 1, 1, None, 256, need, None) == ops.GMM_E_INVALID  # no idx
    assert b(1, 1, 100, 2, 8, float("nan"), 1, 1, None, 256, need, None) == ops.GMM_E_INVALID
    assert b(1, 1, 100, 2, 8, 0.0, 1, 1, None, 256, need - 1, None) == ops.GMM_E_WORKSPACE
    assert b(1, 1, 100, 2, 8, 0.0, 1, 1, None, 257, need, None) == ops.GMM_E_WORKSPACE
    assert b(1, 1, 100, 2, 20000, 0.0, 1, 1, None, 256, need, None) == ops.GMM_E_UNSUPPORTED
    assert b(1, 1, -5, 2, 8, 0.0, 1, 1, None, 256, need, None) == ops.GMM_E_INVALID


def test_kmeans_fit_argument_checks(ops):
    f = ops.lib.gmm_kmeans_fit
    need = ops.workspace_bytes(4, 2)
    assert f(1, 10, 4, 4, 0, 1, 2, -1, 0.0, None, None, 256, need, None) == ops.GMM_E_INVALID
    assert f(1, 10, 4, 4, 0, 1, 2, 3, -1.0, None, None, 256, need, None) == ops.GMM_E_INVALID
    assert f(1, 10, 4, 4, 0, 1, 2, 3, float("inf"), None, None, 256, need, None) == ops.GMM_E_INVALID
    # zero steps: nothing runs, nothing is touched
    done = ops._i32(7)
    assert f(1, 10, 4, 4, 0, 1, 2, 0, 0.0, None, ops.ctypes.byref(done), 256, need, None) == ops.GMM_OK
    assert done.value == 0


def test_bench_refuses_more_than_one_gpu():
    # the bench measures one GPU; asking for more exits with a message
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_hidden_run_time_switches():
    # the library's behaviour is set by its arguments only: no environment
    # variable is read anywhere in its sources
    csrc = os.path.join(ROOT, "gmm_em_amd", "csrc")
    for name in os.listdir(csrc):
        src = open(os.path.join(csrc, name)).read()
        assert "getenv" not in src and "secure_getenv" not in src, name


def test_profile_hook_states(ops):
    # end without begin is an error; begin validates its size; begin/end with
    # no launch in between returns zero counts and releases its events
    f, i = ctypes.c_double, ctypes.c_int32
    a, b, na, nb = f(0), f(0), i(0), i(0)
    refs = (ctypes.byref(a), ctypes.byref(na), ctypes.byref(b), ctypes.byref(nb))
    assert ops.lib.gmm_profile_end(*refs) == ops.GMM_E_INVALID
    assert ops.lib.gmm_profile_begin(0) == ops.GMM_E_INVALID
    assert ops.lib.gmm_profile_begin(1 << 20) == ops.GMM_E_INVALID


def test_binding_constants_match_header(ops):
    # the Python binding's status and arithmetic codes are the header's enums
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    vals = dict((m[0], int(m[1])) for m in re.findall(r"\b(GMM_[A-Z0-9_]+)\s*=\s*(-?\d+)", src))
    for name in ("GMM_ESTEP_FP64", "GMM_ESTEP_INT8_SLICES", "GMM_ESTEP_INT8_SLICES_BOTH",
                 "GMM_ESTEP_INT8_SLICES_MSTEP", "GMM_ESTEP_BF16_SPLIT", "GMM_OK",
                 "GMM_E_INVALID", "GMM_E_WORKSPACE", "GMM_E_UNSUPPORTED", "GMM_E_PARAMS",
                 "GMM_F32", "GMM_BF16"):
        assert getattr(ops, name) == vals[name], name
