"""Stage switching from the discrepancy trace (Hybridiff technical summary,
section 2B): the library's host-side rule against the oracle, bit for bit.

Host code only, so these run without a GPU.  The traces are the seeded
synthetic curves of dpp_synth.relmae_trace (fast fall, flat middle, late rise,
with multiplicative noise), plus degenerate ones."""
import numpy as np
import pytest

import displaced_patch_parallelism_net_amd as dpp
import oracle
from dpp_synth import relmae_trace


def same(d, **kw):
    st, t1, t2 = dpp.dpp_hybrid_schedule(d, **kw)
    so, o1, o2 = oracle.hybrid_schedule(d, **kw)
    assert (t1, t2) == (o1, o2), (t1, t2, o1, o2)
    assert st.dtype == np.int32 and (st == so).all()
    return t1, t2


@pytest.mark.parametrize("T", [20, 50, 1000])
@pytest.mark.parametrize("noise", [0.0, 0.003, 0.02])
def test_matches_oracle_on_synthetic_traces(T, noise):
    seen = set()
    for seed in range(40):
        seen.add(same(relmae_trace(seed, T, noise)) == (T, T))
    assert False in seen       # most traces switch somewhere


@pytest.mark.parametrize("kw", [dict(rho=0.0), dict(rho=1.0), dict(rho=0.1, eps=0.0), dict(eps=0.5),
                                dict(min_warmup=10), dict(min_warmup=10 ** 6)])
def test_matches_oracle_over_parameters(kw):
    for seed in range(20):
        same(relmae_trace(seed, 64, 0.01), **kw)


def test_matches_oracle_on_degenerate_traces():
    assert same(np.array([0.5], np.float32)) == (1, 1)
    assert same(np.full(9, 0.25, np.float32)) == (9, 9)
    assert same((10 - np.arange(10)) * np.float32(0.125)) == (10, 10)
    d = relmae_trace(3, 40, 0.01)
    for idx in ([2], [5, 6], [17], list(range(40))):
        e = d.copy()
        e[idx] = np.nan
        same(e)
    e = d.copy()
    e[0] = np.inf                    # x/0 discrepancy at the first step
    same(e)
    e[10:] = 0.0
    same(e)


def test_validation():
    d = np.ones(4, np.float32)
    st = np.empty(4, np.int32)
    t1, t2 = np.zeros(1, np.int64), np.zeros(1, np.int64)
    L = dpp._lib.LIB

    def call(rel=d.ctypes.data, T=4, rho=0.25, eps=0.02, mw=1, stage=st.ctypes.data, a=t1.ctypes.data,
             b=t2.ctypes.data):
        return L.dpp_hybrid_schedule(rel, T, rho, eps, mw, stage, a, b)

    assert call() == 0
    assert call(rel=None) == -1 and call(stage=None) == -1 and call(a=None) == -1 and call(b=None) == -1
    for bad in (dict(T=0), dict(T=-3), dict(mw=0), dict(rho=-0.1), dict(rho=1.5), dict(rho=float("nan")),
                dict(eps=-0.01), dict(eps=float("nan"))):
        assert call(**bad) == -2, bad
    with pytest.raises(dpp.DppError):
        dpp.dpp_hybrid_schedule(np.zeros(0, np.float32))
