"""Pins of the activation-weighted (AW) search oracle (oracle/aw.py).

The pages give the objective (a search for each group's scale and offset
weighted by E[x^2] of the input channel) but neither a grid nor a tie rule, so
these tests pin the oracle's own specification from outside it: the step-0
candidate and zero importance reduce to RTN, the weighted error never exceeds
RTN's, the choice agrees with an exact rational brute force over the same
candidates, and on activations with massive channels AW lowers the output
error against RTN.
"""

from fractions import Fraction

import numpy as np
import pytest

from gemm_rwkv_amd import synth
from oracle import aw, codecs, quant, ref

SYM = [(8, 16), (8, 64), (4, 16), (4, 32), (4, 64), (6, 32), (5, 64)]


def _weights(n, k, seed):
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)) / np.sqrt(k)
    w[0, :8] *= 6.0          # an outlier-heavy group
    return w.astype(np.float32)


def _importance(k, seed):
    """A nonnegative E[x^2]-like vector: exponential spread, three channels
    2500 times larger (a scale-50 activation's square)."""
    g = np.random.default_rng(seed)
    a = g.exponential(1.0, k)
    a[g.choice(k, 3, replace=False)] = 2500.0
    return a.astype(np.float32)


@pytest.mark.parametrize("bits,group", SYM)
def test_zero_importance_is_rtn(bits, group):
    w = _weights(8, 256, bits + group)
    got = aw.quantize_sym_aw(w, np.zeros(256, np.float32), bits, group)
    want = quant.quantize_sym(w, bits, group)
    assert np.all(got["t"] == 0)
    assert np.array_equal(got["codes"], want["codes"])
    assert np.array_equal(got["scales"].view(np.uint16), want["scales"].view(np.uint16))
    if bits in (5, 6):
        assert np.array_equal(got["hi"], want["hi"])


def test_zero_importance_is_rtn_sb256():
    w = _weights(6, 512, 3)
    got = aw.quantize_sb256_aw(w, np.zeros(512, np.float32))
    want = quant.quantize_sb256(w)
    assert np.all(got["t"] == 0)
    for name in ("qs", "d", "dmin", "sub"):
        assert np.array_equal(np.asarray(got[name]).view(np.uint8), np.asarray(want[name]).view(np.uint8)), name


@pytest.mark.parametrize("bits,group", SYM)
def test_weighted_error_not_above_rtn(bits, group):
    """Recomputed from the returned codes and scales (not from the oracle's
    err array): the chosen weighted error is at most RTN's."""
    n, k = 16, 512
    w = _weights(n, k, 10 + bits + group)
    a = _importance(k, 1).astype(np.float64)
    got = aw.quantize_sym_aw(w, a.astype(np.float32), bits, group)
    rtn = quant.quantize_sym(w, bits, group)
    wd = w.astype(np.float64)

    def err(parts):
        wh = quant.dequant_sym(parts["codes"], parts["scales"], bits, group, parts.get("hi"))
        return np.sum((a * (wd - wh) ** 2).reshape(n, k // group, group), axis=2)

    e_aw, e_rtn = err(got), err(rtn)
    assert np.all(e_aw <= e_rtn * (1 + 1e-9))
    assert np.sum(e_aw) < np.sum(e_rtn)          # the search changes something


def _nearest_code(v, lo, hi):
    """Exact nearest integer in [lo, hi] to the Fraction v, ties to even."""
    f = v.numerator // v.denominator
    r = v - f
    c = f + 1 if (r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2)) else f
    return min(max(c, lo), hi)


@pytest.mark.parametrize("bits,group", [(4, 16), (8, 16), (4, 32), (6, 32), (5, 32)])
def test_sym_choice_matches_exact_bruteforce(bits, group):
    """Each candidate's error computed exactly in rationals (codes by exact
    nearest-integer rounding of w / s_t); the smallest t within the tie factor
    of the exact minimum must be the oracle's choice."""
    n, k = 6, 2 * group
    w = _weights(n, k, 20 + bits)
    a = _importance(k, 2)
    got = aw.quantize_sym_aw(w, a, bits, group)
    Q = (1 << (bits - 1)) - 1
    tie = 1 + Fraction(aw.AW_TIE)
    for i in range(n):
        for gi in range(k // group):
            ws = [Fraction(float(v)) for v in w[i, gi * group:(gi + 1) * group]]
            As = [Fraction(float(v)) for v in a[gi * group:(gi + 1) * group]]
            base = max(abs(v) for v in ws) / Q
            errs = []
            for t in range(aw.AW_STEPS):
                # the candidate scale: fp16 of the fp64 product, as specified
                st = float(codecs.f16_encode(np.float64(float(base)) * (1.0 - t / 32.0)))
                s = Fraction(st)
                e = Fraction(0)
                for wv, av in zip(ws, As):
                    q = 0 if s == 0 else _nearest_code(wv / s, -Q, Q)
                    e += av * (wv - q * s) ** 2
                errs.append(e)
            emin = min(errs)
            want = next(t for t, e in enumerate(errs) if e <= emin * tie)
            assert got["t"][i, gi] == want, (i, gi, got["t"][i, gi], want)


def test_sb256_choice_matches_exact_bruteforce():
    n, k = 3, 256
    w = _weights(n, k, 31)
    a = _importance(k, 3)
    got = aw.quantize_sb256_aw(w, a)
    tie = 1 + Fraction(aw.AW_TIE)
    for i in range(n):
        for j in range(8):
            seg = w[i, 32 * j:32 * (j + 1)].astype(np.float64)
            As = [Fraction(float(v)) for v in a[32 * j:32 * (j + 1)]]
            hi = float(np.max(seg))
            lo = min(0.0, float(np.min(seg)))
            errs = []
            for t in range(aw.AW_STEPS):
                f = 1.0 - t / 32.0
                lo_t, hi_t = lo * f, hi * f          # fp64, as specified
                s = Fraction((hi_t - lo_t) / 15.0)
                m = Fraction(0.0 - lo_t)
                e = Fraction(0)
                for wv, av in zip(seg, As):
                    wq = Fraction(float(wv))
                    u = 0 if s == 0 else _nearest_code((wq + m) / s, 0, 15)
                    e += av * (wq - (s * u - m)) ** 2
                errs.append(e)
            emin = min(errs)
            want = next(t for t, e in enumerate(errs) if e <= emin * tie)
            assert got["t"][i, 0, j] == want, (i, j, got["t"][i, 0, j], want)


@pytest.mark.parametrize("fmt,group", [(quant.W4_SYM, 64), (quant.W4_ASYM_SB256, 32), (quant.W8_SYM, 16)])
def test_aw_lowers_output_error_on_massive_channels(fmt, group):
    """The News page's point: on inputs whose energy sits in a few channels, the
    E[x^2]-weighted choice lowers the error of y = x W^T against RTN.  The
    importance comes from a calibration batch; the error is measured on a
    held-out batch of the same generator."""
    n, k = 64, 2560
    w = synth.weight(2, 0, synth.MAT_O, n, k)
    xc = synth.act_massive(256, k, cfg=2, salt=5).astype(np.float64)
    a = np.mean(xc * xc, axis=0).astype(np.float32)
    x = synth.act_massive(64, k, cfg=2, salt=6)
    y_fp = x.astype(np.float64) @ w.astype(np.float64).T
    p_rtn = quant.quantize(w, fmt, group)
    p_aw = aw.quantize_aw(w, a, fmt, group)
    y_rtn, _ = ref.weight_only_ref(x, fmt, p_rtn, group)
    y_aw, _ = ref.weight_only_ref(x, fmt, p_aw, group)
    e_rtn = np.linalg.norm(y_rtn - y_fp)
    e_aw = np.linalg.norm(y_aw - y_fp)
    assert e_aw < 0.9 * e_rtn, (e_aw, e_rtn)


def test_importance_validation():
    w = _weights(2, 64, 0)
    with pytest.raises(ValueError):
        aw.quantize_sym_aw(w, np.full(64, -1.0, np.float32), 4, 64)
    with pytest.raises(ValueError):
        aw.quantize_sym_aw(w, np.full(64, np.nan, np.float32), 4, 64)
    with pytest.raises(ValueError):
        aw.quantize_sym_aw(w, np.ones(32, np.float32), 4, 64)
