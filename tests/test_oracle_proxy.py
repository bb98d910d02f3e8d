"""Pins of the RWKVQuant proxy oracle (oracle/proxy.py) against closed forms.

Sources: "RWKVQuant: Quantizing the RWKV Family with Proxy Guided Hybrid of
Scalar and Vector Quantization", Abstract (index page) and
pith_extraction.key_machinery (machine-review page).  The readings the oracle
takes where the pages are silent (gaps normalised by their mean, entropy of
the gaps as a distribution in nats, K = 4, v_k = 1/k!) are stated in its
header; every value below follows from those readings by hand or from a
textbook limit, not from the oracle's code:

* a uniform grid of weights has P_c = 0 and every central moment 0;
* gaps alternating a and b: with d = (a - b) / (a + b) the normalised gaps
  are 1 +- d, so M_k = d^k (k even), 0 (k odd), and
  P_c = ((1 + d) log(1 + d) + (1 - d) log(1 - d)) / 2;
* n - 1 unit gaps and one of length L (S = n - 1 + L):
  P_c = log(n / S) + (L / S) log L and
  M_k = ((n - 1) ((1 - L) / S)^k + ((n - 1) (L - 1) / S)^k) / n;
* i.i.d. U(0, 1) weights: the normalised spacings tend to Exp(1), whose
  central moments are 1, 2, 9 (k = 2, 3, 4) and for which
  log n - H -> E[X log X] = 1 - Euler's gamma;
* a hand-worked tensor with repeated values (zero gaps);
* invariance under permutation and under w -> a w + b (a > 0).
"""

import math

import numpy as np
import pytest

from oracle import proxy

EULER_GAMMA = 0.5772156649015329


def _shuffled(s, seed):
    g = np.random.default_rng(seed)
    return g.permutation(np.asarray(s, dtype=np.float64))


def _from_gaps(G, seed=0):
    return _shuffled(np.concatenate([[0.0], np.cumsum(G)]) - 3.0, seed)


def test_uniform_grid_is_zero():
    w = _shuffled(0.25 * np.arange(4097) - 7.0, 1)
    pc, pf, mk = proxy.proxy(w, K=6)
    assert abs(pc) < 1e-12
    assert np.all(np.abs(mk) < 1e-24)
    assert pf < 1e-24


@pytest.mark.parametrize("a,b,n", [(1.0, 3.0, 1000), (0.5, 0.25, 64), (2.0, 2.0, 10)])
def test_two_level_gaps(a, b, n):
    G = np.array([a, b] * (n // 2))
    w = _from_gaps(G, n)
    d = (a - b) / (a + b)
    K = 6
    pc, pf, mk = proxy.proxy(w, K=K)
    want_mk = np.array([d ** k if k % 2 == 0 else 0.0 for k in range(2, K + 1)])
    want_pc = 0.5 * ((1 + d) * math.log(1 + d) + ((1 - d) * math.log(1 - d) if d != 1 else 0.0))
    want_pf = sum(abs(want_mk[k - 2]) / math.factorial(k) for k in range(2, K + 1))
    assert pc == pytest.approx(want_pc, abs=1e-10)
    assert np.allclose(mk, want_mk, atol=1e-10)
    assert pf == pytest.approx(want_pf, abs=1e-10)


@pytest.mark.parametrize("n,L", [(100, 50.0), (1000, 1000.0), (64, 0.1), (300, 0.0)])
def test_single_outlier_gap(n, L):
    G = np.ones(n)
    G[n // 3] = L
    w = _from_gaps(G, 7)
    S = n - 1 + L
    want_pc = math.log(n / S) + ((L / S) * math.log(L) if L > 0 else 0.0)
    want_mk = np.array([((n - 1) * ((1 - L) / S) ** k + ((n - 1) * (L - 1) / S) ** k) / n for k in range(2, 5)])
    pc, pf, mk = proxy.proxy(w)
    assert pc == pytest.approx(want_pc, abs=1e-10)
    assert np.allclose(mk, want_mk, rtol=1e-9, atol=1e-12)
    assert pf == pytest.approx(abs(want_mk[0]) / 2 + abs(want_mk[1]) / 6 + abs(want_mk[2]) / 24, rel=1e-9)
    if L < 1:
        assert mk[1] < 0  # a short gap skews the gaps left: the |.| matters


def test_outlier_grows_fine_proxy():
    vals = []
    for L in (1.0, 5.0, 50.0, 500.0):
        G = np.ones(512)
        G[100] = L
        vals.append(proxy.fine(_from_gaps(G)))
    assert vals[0] < 1e-24 and all(x < y for x, y in zip(vals, vals[1:]))


def test_uniform_samples_tend_to_exponential_spacings():
    w = np.random.default_rng(11).random(1 << 20)
    pc, pf, mk = proxy.proxy(w)
    # standard errors over n = 2^20 spacings: about 0.003, 0.016, 0.12
    assert mk[0] == pytest.approx(1.0, abs=0.015)
    assert mk[1] == pytest.approx(2.0, abs=0.08)
    assert mk[2] == pytest.approx(9.0, abs=0.6)
    assert pc == pytest.approx(1.0 - EULER_GAMMA, abs=0.01)
    assert pf == pytest.approx(1 / 2 + 2 / 6 + 9 / 24, abs=0.04)
    # so near-uniform weights route to scalar quantization under the RWKV-7
    # thresholds, and Gaussian ones (long tails: large gaps far from the mean
    # gap) to vector quantization
    assert proxy.route(pc, pf) == "SQ"
    z = np.random.default_rng(12).standard_normal(1 << 18)
    assert proxy.route(*proxy.proxy(z)[:2]) == "VQ"


def test_hand_example_with_repeated_weights():
    # sorted 0,0,1,1,2,2: gaps 0,1,0,1,0 (mean 0.4) -> g = 0, 2.5, 0, 2.5, 0;
    # p = 0, 1/2, 0, 1/2, 0 so H = log 2 and P_c = log 5 - log 2;
    # g - 1 = -1, 1.5, -1, 1.5, -1: M2 = 7.5/5, M3 = 3.75/5, M4 = 13.125/5;
    # P_f = 1.5/2 + 0.75/6 + 2.625/24 = 0.984375
    w = np.array([2.0, 0.0, 1.0, 2.0, 0.0, 1.0])
    pc, pf, mk = proxy.proxy(w)
    assert pc == pytest.approx(math.log(2.5), abs=1e-15)
    assert np.allclose(mk, [1.5, 0.75, 2.625], atol=1e-15)
    assert pf == pytest.approx(0.984375, abs=1e-15)
    assert proxy.proxy(w, K=3, v=[2.0, -1.0])[1] == pytest.approx(2 * 1.5 - 0.75, abs=1e-15)


def test_invariances():
    g = np.random.default_rng(5)
    w = g.standard_normal(20000) * np.exp(g.standard_normal(20000))
    base = proxy.proxy(w, K=5)
    for t in (g.permutation(w), 3.5 * w - 2.0, 1e-3 * w + 7.0):
        got = proxy.proxy(t, K=5)
        assert got[0] == pytest.approx(base[0], rel=1e-7, abs=1e-9)
        assert got[1] == pytest.approx(base[1], rel=1e-6)
        assert np.allclose(got[2], base[2], rtol=1e-6)


def test_route_and_degenerate_inputs():
    assert proxy.route(0.0, 0.0) == "SQ"
    assert proxy.route(1.54, 0.0) == "VQ" and proxy.route(0.0, 30.0) == "VQ"
    assert proxy.route(1.53, 29.9) == "SQ"
    for bad in ([1.0, 2.0], np.full(10, 3.0), [0.0, np.nan, 1.0], [0.0, np.inf, 1.0]):
        with pytest.raises(ValueError):
            proxy.proxy(bad)
    with pytest.raises(ValueError):
        proxy.proxy(np.arange(10.0), K=4, v=[1.0, 1.0])


# planted mistakes: each must break at least one pin above

def _pins_fail():
    checks = [test_uniform_grid_is_zero, test_hand_example_with_repeated_weights, test_invariances,
              lambda: test_two_level_gaps(1.0, 3.0, 1000), lambda: test_single_outlier_gap(64, 0.1)]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    return failed


def test_mutation_raw_gaps(monkeypatch):
    def raw(w):
        s = np.sort(np.asarray(w, dtype=np.float64).ravel())
        return np.diff(s)
    monkeypatch.setattr(proxy, "gaps", raw)
    assert _pins_fail() > 0


def test_mutation_entropy_in_bits(monkeypatch):
    def h2(g):
        p = g / g.sum()
        nz = p[p > 0]
        return float(-(nz * np.log2(nz)).sum())
    monkeypatch.setattr(proxy, "entropy", h2)
    assert _pins_fail() > 0


def test_mutation_signed_moments(monkeypatch):
    # |M_k| dropped: the negative third moment of left-skewed gaps then subtracts
    def signed(w, K=4, v=None):
        g = proxy.gaps(w)
        v = proxy.default_weights(K) if v is None else np.asarray(v, dtype=np.float64)
        mk = proxy.central_moments(g, K)
        return math.log(g.size) - proxy.entropy(g), float(np.sum(v * mk)), mk
    monkeypatch.setattr(proxy, "proxy", signed)
    with pytest.raises(AssertionError):
        test_single_outlier_gap(64, 0.1)
