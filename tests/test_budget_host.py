"""KL-budget schedule and mismatch-subtracted effective budget: the library's host
functions against the oracle ([paper] App. D.1 "KL budget", Table 4; [summary] D.1).
Host-only calls, no GPU needed."""
import ctypes
import math
import os

import pytest

import oracle
from rank_gradient_sketching_logra_amd import binding as B


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(B.LIB_PATH):
        import rank_gradient_sketching_logra_amd.build as build
        build.build(verbose=False)
    B.lib()


def test_schedule_matches_oracle():
    for H, dmax, dmin in ((300, 2e-4, 2e-5), (1000, 2e-4, 2e-5), (2, 1.0, 0.5), (7, 3e-3, 0.0)):
        for u in list(range(1, H + 3)) + [5 * H]:
            got = B.kl_budget(u, H, dmax, dmin)
            want = oracle.kl_budget(u, H, dmax, dmin)
            assert got == pytest.approx(want, rel=1e-15, abs=0.0), (H, u)


def test_mismatch_ema_and_effective_budget_match_oracle():
    seq = [None, float("nan"), 3e-5, -1e-5, 2e-5, float("nan"), 8e-5, 0.0, 1e-4, None, 4e-6]
    st = B.MismatchState(0.0, 0, 0)
    kappa = None
    for u, m in enumerate(seq, start=1):
        B.mismatch_update(st, m, 0.3)
        kappa = oracle.mismatch_ema(kappa, m, 0.3)
        assert bool(st.valid) == (kappa is not None)
        if kappa is not None:
            assert st.kappa == pytest.approx(kappa, rel=1e-15, abs=0.0)
            assert st.kappa >= 0.0
        du = oracle.kl_budget(u, 300, 2e-4, 2e-5)
        got = B.effective_budget(du, st)
        assert got == pytest.approx(oracle.effective_budget(du, kappa), rel=1e-15, abs=0.0)
        assert got >= 0.5 * du                       # the 50% floor


def test_budget_argument_errors():
    lib = B.lib()
    out = ctypes_double()
    assert lib.logra_kl_budget(0, 300, 2e-4, 2e-5, out) == B.ERR_DOMAIN
    assert lib.logra_kl_budget(1, 1, 2e-4, 2e-5, out) == B.ERR_DOMAIN
    assert lib.logra_kl_budget(1, 300, 2e-5, 2e-4, out) == B.ERR_DOMAIN      # max < min
    assert lib.logra_kl_budget(1, 300, math.inf, 2e-5, out) == B.ERR_DOMAIN
    assert lib.logra_kl_budget(1, 300, 2e-4, 2e-5, None) == B.ERR_NULL
    st = B.MismatchState(0.0, 0, 0)
    assert lib.logra_mismatch_update(ctypes.byref(st), 1e-5, 0.0) == B.ERR_DOMAIN
    assert lib.logra_mismatch_update(ctypes.byref(st), math.inf, 0.3) == B.ERR_DOMAIN
    assert lib.logra_mismatch_update(None, 1e-5, 0.3) == B.ERR_NULL
    assert lib.logra_effective_budget(-1.0, ctypes.byref(st), out) == B.ERR_DOMAIN
    assert lib.logra_effective_budget(1e-4, None, out) == B.ERR_NULL


def ctypes_double():
    return ctypes.byref(ctypes.c_double(0.0))
