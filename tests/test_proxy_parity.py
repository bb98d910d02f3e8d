"""The library's RWKVQuant proxy (rq_proxy, host code in librq) against the
oracle (oracle/proxy.py) on the same seeded weights: synthetic projections of
the RWKV-7 widths, weights with massive columns, ragged and tiny tensors,
repeated values, other K and v, and the error paths.  Both compute in fp64
from the same fp32 weights; the tolerance covers summation order only."""

import numpy as np
import pytest

from gemm_rwkv_amd import rq, synth
from oracle import proxy

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(rq._LIB_PATH), reason="librq not built")


def _close(got, want, K):
    assert got[0] == pytest.approx(want[0], rel=1e-10, abs=1e-12)
    assert got[1] == pytest.approx(want[1], rel=1e-9, abs=1e-12)
    assert np.allclose(got[2], want[2], rtol=1e-9, atol=1e-12)
    assert len(got[2]) == K - 1


@pytest.mark.parametrize("c", [768, 2048])
def test_layer_weights(c):
    for mat, n, k in synth.layer_shapes(c):
        w = synth.weight(0, 17, mat, n, k)
        _close(rq.rq_proxy(w), proxy.proxy(w), 4)


def test_massive_columns_and_heavy_tails():
    g = np.random.default_rng(3)
    w = (g.standard_normal((512, 1024)) / 32).astype(np.float32)
    w[:, [5, 700]] *= 40.0
    t = (g.standard_t(2, 300001)).astype(np.float32)
    for a in (w, t):
        _close(rq.rq_proxy(a), proxy.proxy(a.astype(np.float64)), 4)


@pytest.mark.parametrize("count", [3, 4, 5, 17, 1000, 65537])
@pytest.mark.parametrize("K", [2, 3, 4, 8, 16])
def test_ragged_sizes_and_orders(count, K):
    w = np.random.default_rng(count * 31 + K).standard_normal(count).astype(np.float32)
    _close(rq.rq_proxy(w, K=K), proxy.proxy(w, K=K), K)


def test_repeated_values_and_custom_weights():
    w = np.repeat(np.arange(-20, 21, dtype=np.float32) * 0.125, 7)
    _close(rq.rq_proxy(w), proxy.proxy(w), 4)
    v = [0.5, -2.0, 3.0, 0.25]
    _close(rq.rq_proxy(w, K=5, v=v), proxy.proxy(w, K=5, v=v), 5)
    # the hand-worked example of the oracle's pins
    pc, pf, mk = rq.rq_proxy(np.array([2, 0, 1, 2, 0, 1], np.float32))
    assert pc == pytest.approx(np.log(2.5), abs=1e-14) and pf == pytest.approx(0.984375, abs=1e-14)


def test_uniform_grid_and_routing():
    w = np.random.default_rng(0).permutation(np.arange(8192, dtype=np.float32) * 0.5 - 100.0)
    pc, pf, mk = rq.rq_proxy(w)
    assert abs(pc) < 1e-12 and pf < 1e-24
    assert rq.proxy_route(pc, pf) == "SQ" == proxy.route(pc, pf)
    assert rq.proxy_route(2.0, 0.0) == "VQ" and rq.proxy_route(0.0, 31.0) == "VQ"


def test_errors():
    L = rq.lib()
    import ctypes
    d = ctypes.c_double()
    ok = np.arange(8, dtype=np.float32)
    assert L.rq_proxy(None, 8, 4, None, ctypes.addressof(d), ctypes.addressof(d), None) == rq.RQ_ERR_NULL
    assert L.rq_proxy(ok.ctypes.data, 8, 4, None, None, ctypes.addressof(d), None) == rq.RQ_ERR_NULL
    for count, K in ((2, 4), (8, 1), (8, rq.RQ_PROXY_MAX_K + 1)):
        assert L.rq_proxy(ok.ctypes.data, count, K, None, ctypes.addressof(d), ctypes.addressof(d), None) == \
            rq.RQ_ERR_SHAPE
    bad = ok.copy()
    bad[3] = np.inf
    assert L.rq_proxy(bad.ctypes.data, 8, 4, None, ctypes.addressof(d), ctypes.addressof(d), None) == \
        rq.RQ_ERR_NONFINITE
    const = np.full(9, 1.5, np.float32)
    assert L.rq_proxy(const.ctypes.data, 9, 4, None, ctypes.addressof(d), ctypes.addressof(d), None) == \
        rq.RQ_ERR_DEGENERATE
    with pytest.raises(rq.RqError):
        rq.rq_proxy(const)
