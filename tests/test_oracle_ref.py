"""Pins for the oracle's reference products and comparator (CPU only).

* The fp64 product against exact rational sums on tiny inputs (catches a
  transposed operand or a wrong index) and against unit-vector probes.
* Integer special cases whose exact value is known in closed form: codes with
  a +-Q entry per group get scale 1, so y is the integer matrix-vector product.
* The comparator on planted errors just inside and just outside the bound.
* The synthetic input generators against the figures the pages print.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from gemm_rwkv_amd import synth
from oracle import codecs, quant, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_matmul_ref_exact_small():
    g = np.random.default_rng(0)
    x = g.standard_normal((3, 7))
    w = g.standard_normal((4, 7))
    y, b = ref.matmul_ref(x, w)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(7))
            absb = sum(abs(Fraction(float(x[m, k])) * Fraction(float(w[n, k]))) for k in range(7))
            assert abs(Fraction(float(y[m, n])) - exact) <= absb * Fraction(8, 2 ** 53)
            assert abs(Fraction(float(b[m, n])) - absb) <= absb * Fraction(1, 2 ** 50)


def test_matmul_ref_unit_vectors():
    g = np.random.default_rng(1)
    w = g.standard_normal((5, 9))
    eye = np.eye(9)
    y, _ = ref.matmul_ref(eye, w)
    assert np.array_equal(y, w.T)       # y[k][n] = w[n][k]
    with pytest.raises(ValueError):
        ref.matmul_ref(np.ones((1, 8)), w)


@pytest.mark.parametrize("fmt,bits", [(quant.W4_SYM, 4), (quant.W8_SYM, 8)])
@pytest.mark.parametrize("group", [16, 32, 64])
def test_weight_only_integer_closed_form(fmt, bits, group):
    g = np.random.default_rng(group + bits)
    Q = (1 << (bits - 1)) - 1
    n, k = 6, 4 * group
    q = g.integers(-Q, Q + 1, (n, k))
    q[:, ::group] = Q                       # absmax Q in every group -> s = 1
    x = g.integers(-3, 4, (2, k))
    parts = quant.quantize(q.astype(np.float32), fmt, group)
    assert np.all(parts["scales"] == 1.0)
    y, b = ref.weight_only_ref(x.astype(np.float16), fmt, parts, group)
    want = [[sum(int(x[m, kk]) * int(q[nn, kk]) for kk in range(k)) for nn in range(n)] for m in range(2)]
    assert y.tolist() == want
    wantb = [[sum(abs(int(x[m, kk]) * int(q[nn, kk])) for kk in range(k)) for nn in range(n)] for m in range(2)]
    assert b.tolist() == wantb


def test_sb256_integer_closed_form():
    # d = dmin = 1, sc = 1, mc = 8: w_hat = q - 8 exactly
    g = np.random.default_rng(4)
    n, k = 3, 512
    q = g.integers(0, 16, (n, k))
    q[:, ::32] = 0
    q[:, 1::32] = 15
    w = (q - 8).astype(np.float32)
    # one group per superblock with range [-63, 0] pins dmin = 1 and another
    # with range 63*15 pins d = 1; skip that and build the parts directly
    parts = {"qs": quant.pack_nibbles(q),
             "d": np.ones((n, 2), np.float16), "dmin": np.ones((n, 2), np.float16),
             "sub": quant.pack_sub(np.ones((n, 2, 8), np.uint8), np.full((n, 2, 8), 8, np.uint8))}
    x = g.integers(-2, 3, (1, k))
    y, _ = ref.weight_only_ref(x.astype(np.float16), quant.W4_ASYM_SB256, parts)
    assert y[0].tolist() == [int(np.dot(x[0].astype(np.int64), (q[i] - 8).astype(np.int64))) for i in range(n)]
    assert np.array_equal(quant.dequant(quant.W4_ASYM_SB256, parts), w.astype(np.float64))


def test_w8a8_integer_closed_form():
    g = np.random.default_rng(6)
    # integer-valued e4m3fn operands, absmax 448 per row -> unit scales
    ints = np.array([v for v in codecs.E4M3_TABLE[:0x7F] if v == int(v) and v <= 16])
    x = g.choice(np.concatenate([ints, -ints]), (4, 128))
    w = g.choice(np.concatenate([ints, -ints]), (5, 128))
    x[:, 0] = 448.0
    w[:, 0] = -448.0
    xq = quant.quantize_rows(x.astype(np.float32), "fp8")
    wq = quant.quantize(w.astype(np.float32), quant.FP8_E4M3_CH)
    assert np.all(xq["scales"] == 1) and np.all(wq["scales"] == 1)
    y, _ = ref.w8a8_ref(xq["codes"], xq["scales"], "fp8", quant.FP8_E4M3_CH, wq)
    assert y.tolist() == (x.astype(np.int64) @ w.astype(np.int64).T).tolist()


def check_w8a8_int8_closed_form(as_bytes):
    """int8 W8A8: rows whose absmax is 127 * 2**e get the exact scale 2**e
    (Toolkit page, Key Design: int8 x int8 products with one scale per token
    and per output channel), so y = s_x[m] * s_w[n] * (integer dot product)
    exactly.  Codes are passed as signed int8 or as the raw bytes a device
    buffer holds; -127 and 127 sit in every row."""
    g = np.random.default_rng(11)
    xi = g.integers(-127, 128, (4, 96))
    wi = g.integers(-127, 128, (6, 96))
    xi[:, 0], xi[:, 1] = 127, -127
    wi[:, 0], wi[:, 1] = -127, 127
    ex = g.integers(-6, 7, 4)
    ew = g.integers(-6, 7, 6)
    x = (xi * np.exp2(ex)[:, None]).astype(np.float32)
    w = (wi * np.exp2(ew)[:, None]).astype(np.float32)
    xq = quant.quantize_rows(x, "int8")
    wq = quant.quantize(w, quant.I8_CH)
    assert np.array_equal(xq["codes"].astype(np.int64), xi)
    assert np.array_equal(wq["codes"].astype(np.int64), wi)
    assert np.array_equal(xq["scales"], np.exp2(ex).astype(np.float32))
    codes = xq["codes"].view(np.uint8) if as_bytes else xq["codes"]
    if as_bytes:
        wq = dict(wq, codes=wq["codes"].view(np.uint8))
    y, b = ref.w8a8_ref(codes, xq["scales"], "int8", quant.I8_CH, wq)
    want = [[float(sum(int(xi[m, k]) * int(wi[n, k]) for k in range(96))) * 2.0 ** (int(ex[m]) + int(ew[n]))
             for n in range(6)] for m in range(4)]
    assert y.tolist() == want
    bw = [[float(sum(abs(int(xi[m, k]) * int(wi[n, k])) for k in range(96))) * 2.0 ** (int(ex[m]) + int(ew[n]))
           for n in range(6)] for m in range(4)]
    assert b.tolist() == bw


@pytest.mark.parametrize("as_bytes", [False, True])
def test_w8a8_int8_closed_form(as_bytes):
    check_w8a8_int8_closed_form(as_bytes)


def test_mutation_int8_codes_read_unsigned(monkeypatch):
    """Reading the int8 activation codes as unsigned bytes (a plausible slip
    in dequant_rows) must fail the closed form above."""
    def unsigned(codes, scales, kind):
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]
        if kind == "fp8":
            return codecs.e4m3_decode(codes) * s
        return np.asarray(codes).view(np.uint8).astype(np.float64) * s
    monkeypatch.setattr(quant, "dequant_rows", unsigned)
    with pytest.raises(AssertionError):
        check_w8a8_int8_closed_form(True)


def test_int_acc_ref():
    g = np.random.default_rng(8)
    a = g.integers(-127, 128, (3, 40)).astype(np.int8)
    b = g.integers(-127, 128, (4, 40)).astype(np.int8)
    acc = ref.int_acc_ref(a, b)
    for m in range(3):
        for n in range(4):
            assert acc[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(40))
    # worst case of the largest configured K stays inside int32
    assert 127 * 127 * 16384 < 2 ** 31


def test_compare_bounds():
    y_ref = np.array([[1.0, -2.0, 0.0, 100.0]])
    b = np.array([[2.0, 3.0, 0.0, 150.0]])
    tol = 2e-3 * b + 1e-3
    ok, info = ref.compare(y_ref.copy(), y_ref, b)
    assert ok and info["max_ratio"] == 0
    y = y_ref + 0.99 * tol
    y[0, 3] = y_ref[0, 3]                      # keep L2 small
    ok, info = ref.compare(y, y_ref, b)
    assert info["max_ratio"] <= 1
    y = y_ref.copy()
    y[0, 0] += 1.01 * tol[0, 0]
    ok, info = ref.compare(y, y_ref, b)
    assert not ok and info["max_ratio"] > 1
    y = y_ref.copy()
    y[0, 1] = np.nan
    ok, info = ref.compare(y, y_ref, b)
    assert not ok and info["nonfinite"] == 1
    # L2 criterion: errors uniformly at 0.9 of the per-element bound on large
    # outputs fail the 1e-3 relative-L2 test
    y_ref = np.full((1, 100), 10.0)
    b = np.full((1, 100), 10.0)
    y = y_ref + 0.9 * (2e-3 * b + 1e-3)
    ok, info = ref.compare(y, y_ref, b)
    assert info["max_ratio"] < 1 and info["rel_l2"] > 1e-3 and not ok


def check_square_integer_product():
    g = np.random.default_rng(9)
    x = g.integers(-5, 6, (2, 6))
    w = g.integers(-5, 6, (6, 6))
    y, _ = ref.matmul_ref(x.astype(np.float64), w.astype(np.float64))
    want = [[sum(int(x[m, k]) * int(w[n, k]) for k in range(6)) for n in range(6)] for m in range(2)]
    assert y.tolist() == want


def test_square_integer_product():
    check_square_integer_product()


def test_mutation_transposed_weight(monkeypatch):
    real = ref.matmul_ref

    def transposed(xhat, what):
        return real(xhat, np.asarray(what).T.copy())
    monkeypatch.setattr(ref, "matmul_ref", transposed)
    with pytest.raises(AssertionError):
        check_square_integer_product()


# --------------------------------------------------------------------------
# the synthetic generators against the pages' figures
# --------------------------------------------------------------------------


def _fig():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


def test_sizes_table():
    fig = _fig()["rwkv7_sizes"]
    for k, v in fig.items():
        if k.startswith("_"):
            continue
        assert tuple(v) == synth.RWKV7_SIZES[k]


def test_massive_channels():
    fig = _fig()["massive_channels"]
    ch = synth.massive_channels(2560)
    assert fig["2.9B_channel"] in ch and len(ch) == fig["2.9B_count"]
    x = synth.act_massive(16, 2560).astype(np.float64)
    e_all = np.sum(x * x, axis=1)
    e_ch = np.sum(x[:, ch] ** 2, axis=1)
    frac = e_ch / e_all
    # exact before the fp16 cast; fp16 rounding moves it by < 1e-3
    assert np.all(np.abs(frac - fig["2.9B_energy_fraction"]) < 1e-3)
    x10 = synth.act_massive(4, 10240).astype(np.float64)
    ch10 = synth.massive_channels(10240)
    assert 517 in ch10
    assert np.all(np.abs(np.sum(x10[:, ch10] ** 2, 1) / np.sum(x10 ** 2, 1) - 0.98) < 1e-3)
    x1 = synth.act_channel_1202(8, 2048).astype(np.float64)
    assert np.all(np.argmax(np.abs(x1).mean(0)) == _fig()["massive_channels"]["1.5B_channel"])


def test_generators_deterministic():
    a = synth.fused_rkv_768()
    b = synth.fused_rkv_768()
    for u, v in zip(a[0], b[0]):
        assert np.array_equal(u, v)
    assert np.array_equal(a[1], b[1])
    assert a[0][0].dtype == np.float32 and a[1].dtype == np.float16 and a[1].shape == (1, 768)
    assert abs(np.std(a[0][0]) * np.sqrt(768) - 1) < 0.01
    w = synth.weight(1, 0, synth.MAT_KEY, 8192, 2048)
    assert w.shape == (8192, 2048) and abs(np.std(w) * np.sqrt(2048) - 1) < 0.01
    assert not np.array_equal(synth.weight(1, 0, 0, 4, 8), synth.weight(1, 1, 0, 4, 8))
