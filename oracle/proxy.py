"""RWKVQuant's weights-only coarse-to-fine proxy, written out in fp64
(TEST INFRASTRUCTURE: only the test suite may call it).

Source: "RWKVQuant: Quantizing the RWKV Family with Proxy Guided Hybrid of
Scalar and Vector Quantization" -- the arXiv index page, Abstract (a
coarse-to-fine proxy that assesses the uniformity of the weights and finds
their outliers), and the machine-review page of the same paper,
pith_extraction.key_machinery (the weights are flattened and sorted and turned
into adjacent gaps G'; the coarse proxy is the entropy gap
P_c = H(G'^) - H(G') between uniform gaps G'^ and the observed ones; the fine
proxy is P_f = sum_{k=2..K} v_k |M_k| over the central moments M_k of G'; a
layer takes scalar quantization only when P_c < tau_c and P_f < tau_f, with
tau_c = 1.54 and tau_f = 30 reported for RWKV-7 under its falsifier).

The pages leave four steps open; the readings taken here (and by the library):

1. Gaps are normalised by their mean, g_i = G_i / mean(G), i = 1..n with
   n = M - 1 gaps of the M sorted weights, so that a uniform grid has every
   g_i = 1 and both proxies are unchanged by w -> a w + b (a > 0).
2. H(G') is the Shannon entropy (natural log) of the gaps taken as a
   distribution, p_i = g_i / sum(g) = G_i / sum(G), with 0 log 0 = 0.  No
   histogram or binning is involved.  The uniform gaps G'^ have p_i = 1/n, so
   H(G'^) = log n and P_c = log n - H(G') >= 0, zero only for a uniform grid.
3. M_k is the k-th central moment of the normalised gaps,
   M_k = (1/n) sum_i (g_i - 1)^k (their mean is exactly 1).
4. K = 4 and v_k = 1/k! (the coefficients of the Taylor expansion the review
   credits for the fine proxy) unless given.

A tensor needs at least three weights and two distinct values: with all
weights equal the mean gap is zero and the normalisation is undefined.
"""

import math

import numpy as np

TAU_C = 1.54  # coarse threshold reported for RWKV-7
TAU_F = 30.0  # fine threshold reported for RWKV-7


def default_weights(K):
    """v_k = 1/k! for k = 2..K (reading 4)."""
    return np.array([1.0 / math.factorial(k) for k in range(2, K + 1)], dtype=np.float64)


def gaps(w):
    """Adjacent gaps of the flattened, sorted weights, divided by their mean."""
    s = np.sort(np.asarray(w, dtype=np.float64).ravel())
    if s.size < 3:
        raise ValueError("the proxy needs at least three weights")
    if not np.all(np.isfinite(s)):
        raise ValueError("non-finite weight")
    G = np.diff(s)
    mean = G.sum() / G.size
    if mean == 0.0:
        raise ValueError("all weights are equal: the gaps cannot be normalised")
    return G / mean


def entropy(g):
    """Shannon entropy (nats) of the gaps taken as a distribution."""
    p = g / g.sum()
    nz = p[p > 0]
    return float(-(nz * np.log(nz)).sum())


def coarse(w):
    """P_c = H(uniform gaps) - H(observed gaps) = log n - H(G')."""
    g = gaps(w)
    return math.log(g.size) - entropy(g)


def central_moments(g, K):
    """M_k = mean((g - mean(g))^k) for k = 2..K."""
    d = g - g.mean()
    return np.array([float(np.mean(d ** k)) for k in range(2, K + 1)], dtype=np.float64)


def fine(w, K=4, v=None):
    """P_f = sum_{k=2..K} v_k |M_k|."""
    g = gaps(w)
    v = default_weights(K) if v is None else np.asarray(v, dtype=np.float64)
    if v.size != K - 1:
        raise ValueError("v needs K - 1 weights (k = 2..K)")
    return float(np.sum(v * np.abs(central_moments(g, K))))


def proxy(w, K=4, v=None):
    """(P_c, P_f, [M_2..M_K]) of one weight tensor."""
    g = gaps(w)
    v = default_weights(K) if v is None else np.asarray(v, dtype=np.float64)
    if v.size != K - 1:
        raise ValueError("v needs K - 1 weights (k = 2..K)")
    mk = central_moments(g, K)
    pc = math.log(g.size) - entropy(g)
    return pc, float(np.sum(v * np.abs(mk))), mk


def route(pc, pf, tau_c=TAU_C, tau_f=TAU_F):
    """Scalar quantization only when both proxies are below their thresholds."""
    return "SQ" if (pc < tau_c and pf < tau_f) else "VQ"
