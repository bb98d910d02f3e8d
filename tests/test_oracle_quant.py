"""Pins for the oracle's quantizers (CPU only).

Each check below is tied to something other than the oracle's own formulas:
  * hand-derived examples (tests/golden/hand_examples.json),
  * brute force: for every weight, every code is tried and the chosen one must
    minimise |w - w_hat(code)| with ties to the even code; every scale is the
    nearest value of its storage type to the exact rational quotient,
  * exact round trips of weights that are representable in the format,
  * code-range invariants and error bounds on adversarial inputs,
  * byte accounting against the model card's checkpoint sizes.
The ``check_*`` helpers raise AssertionError; the mutation tests at the end
plant mistakes in the oracle and require that a pin catches each one.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _adversarial_weights(n, k, seed):
    """fp32 rows mixing scales 1e-8..1e3, zero groups, constant groups, outliers."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)) * 10.0 ** g.uniform(-8, 3, (n, 1))
    w = w.astype(np.float32)
    if n > 3 and k >= 64:
        w[0, :64] = 0.0                      # all-zero groups
        w[1, :32] = 0.37                     # constant positive group
        w[2, :32] = -1.25                    # constant negative group
        w[3, 5] = 1e4                        # outlier
    return w


# --------------------------------------------------------------------------
# hand-derived examples
# --------------------------------------------------------------------------


def test_sym_hand_examples_5_6_bits():
    ex_all = _golden("hand_examples.json")
    for name, bits in (("sym_int6_g32", 6), ("sym_int5_g32", 5)):
        ex = ex_all[name]
        w = np.array([ex["w"]], dtype=np.float32)
        r = quant.quantize_sym(w, bits, ex["group"])
        assert int(codecs.f16_bits(r["scales"])[0, 0]) == int(ex["scale_f16_bits"], 16)
        assert r["q"][0].tolist() == ex["codes"], name
        assert r["codes"][0].tolist() == [int(b, 16) for b in ex["packed_bytes"]], name
        hb = np.ascontiguousarray(r["hi"][0]).view(np.uint8).tolist()
        assert hb == [int(b, 16) for b in ex["hi_bytes"]], name


@pytest.mark.parametrize("name,bits", [("sym_int8_g16", 8), ("sym_int4_g16", 4),
                                       ("sym_int4_scale_one_seventh", 4)])
def test_sym_hand_examples(name, bits):
    ex = _golden("hand_examples.json")[name]
    w = np.array([ex["w"]], dtype=np.float32)
    r = quant.quantize_sym(w, bits, 16)
    assert int(codecs.f16_bits(r["scales"])[0, 0]) == int(ex["scale_f16_bits"], 16)
    assert r["q"][0].tolist() == ex["codes"]
    if "packed_bytes" in ex:
        assert r["codes"][0].tolist() == [int(b, 16) for b in ex["packed_bytes"]]


def test_sb256_sub_bits_hand_examples():
    for case in _golden("hand_examples.json")["sb256_sub_bits"]["cases"]:
        sc = np.array([[case["sc"]]], dtype=np.uint8)
        mc = np.array([[case["mc"]]], dtype=np.uint8)
        got = quant.pack_sub(sc, mc)[0, 0].tolist()
        assert got == [int(b, 16) for b in case["bytes"]]
        sc2, mc2 = quant.unpack_sub(quant.pack_sub(sc, mc))
        assert np.array_equal(sc2, sc) and np.array_equal(mc2, mc)


def test_sb256_sub_bits_bitwise():
    # bit-by-bit construction of the 96-bit stream, independent of the packer
    g = np.random.default_rng(3)
    sc = g.integers(0, 64, (50, 8)).astype(np.uint8)
    mc = g.integers(0, 64, (50, 8)).astype(np.uint8)
    packed = quant.pack_sub(sc[:, None, :], mc[:, None, :])[:, 0, :]
    for r in range(50):
        bits = [0] * 96
        for j in range(8):
            for b in range(6):
                bits[6 * j + b] = (int(sc[r, j]) >> b) & 1
                bits[48 + 6 * j + b] = (int(mc[r, j]) >> b) & 1
        want = [sum(bits[8 * i + b] << b for b in range(8)) for i in range(12)]
        assert packed[r].tolist() == want


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------


def _nearest_f16_exact(q_frac):
    """Brute-force nearest fp16 (ties to even bits) to a non-negative Fraction."""
    best = None
    # search a window of bit patterns around the float estimate
    est = int(codecs.f16_bits(codecs.f16_encode(float(q_frac))).item()) & 0x7FFF
    for b in range(max(0, est - 2), min(0x7C00, est + 3)):
        v = Fraction(float(codecs.f16_from_bits(np.uint16(b))))
        d = abs(v - q_frac)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    if q_frac >= Fraction(65520):
        return 0x7C00
    return best[1]


def check_sym_brute(bits, group, seed, n=24):
    k = 4 * group
    w = _adversarial_weights(n, k, seed)
    r = quant.quantize_sym(w, bits, group)
    Q = (1 << (bits - 1)) - 1
    s = r["scales"].astype(np.float64)
    q = quant.unpack_sym(r["codes"], bits, r.get("hi")).astype(np.int64)
    assert np.array_equal(q, r["q"].astype(np.int64))
    # scale = nearest fp16 to the exact quotient absmax / Q
    wg = w.reshape(n, k // group, group)
    for i in range(n):
        for j in range(k // group):
            a = Fraction(float(np.max(np.abs(wg[i, j].astype(np.float64)))))
            assert int(codecs.f16_bits(r["scales"][i, j])) == _nearest_f16_exact(a / Q), (i, j)
    # codes: nearest among all codes, ties to even
    cand = np.arange(-Q, Q + 1, dtype=np.float64)
    sg = np.repeat(s, group, axis=1)
    dist = np.abs(w.astype(np.float64)[..., None] - cand * sg[..., None])
    best = dist.min(axis=-1, keepdims=True)
    is_best = dist == best
    n_best = is_best.sum(-1)
    pick = np.where(n_best == 1, np.argmax(is_best, -1),
                    np.argmax(is_best & (cand % 2 == 0), -1))
    want = cand[pick].astype(np.int64)
    want = np.where(sg == 0.0, 0, want)
    assert np.array_equal(q, want)


SYM_CASES = [(b, g) for b in (4, 8) for g in (16, 32, 64)] + [(b, g) for b in (5, 6) for g in (32, 64)]


@pytest.mark.parametrize("bits,group", SYM_CASES)
def test_sym_brute_force(bits, group):
    check_sym_brute(bits, group, seed=bits * 100 + group)


def check_rows_brute(kind, seed, n=40, k=96):
    w = _adversarial_weights(n, k, seed)
    r = quant.quantize_rows(w, kind)
    s = r["scales"].astype(np.float64)
    div = 448 if kind == "fp8" else 127
    for i in range(n):
        a = Fraction(float(np.max(np.abs(w[i].astype(np.float64)))))
        # nearest fp32 to a / div: check against both fp32 neighbours
        sv = Fraction(float(s[i]))
        lo = Fraction(float(np.nextafter(np.float32(s[i]), np.float32(0))))
        hi = Fraction(float(np.nextafter(np.float32(s[i]), np.float32(np.inf))))
        t = a / div
        assert abs(sv - t) <= abs(lo - t) and abs(sv - t) <= abs(hi - t)
    if kind == "fp8":
        mags = codecs.E4M3_TABLE[:0x7F]
        for i in range(n):
            for j in range(k):
                if s[i] == 0:
                    assert r["codes"][i, j] == 0
                    continue
                v = float(w[i, j]) / s[i]
                d = np.abs(abs(v) - mags)
                cands = np.nonzero(d == d.min())[0]
                c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
                want = int(c) | (0x80 if np.signbit(v) else 0)
                assert int(r["codes"][i, j]) == want, (i, j, v)
    else:
        cand = np.arange(-127, 128, dtype=np.float64)
        quo = w.astype(np.float64)
        dist = np.abs(quo[..., None] - cand * s[:, None, None])
        best = dist.min(-1, keepdims=True)
        is_best = dist == best
        pick = np.where(is_best.sum(-1) == 1, np.argmax(is_best, -1),
                        np.argmax(is_best & (cand % 2 == 0), -1))
        want = np.where(s[:, None] == 0, 0, cand[pick]).astype(np.int64)
        assert np.array_equal(r["codes"].astype(np.int64), want)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_rows_brute_force(kind):
    check_rows_brute(kind, seed=7 if kind == "fp8" else 8)


def check_sb_brute(seed, n=6, k=512):
    w = _adversarial_weights(n, k, seed)
    r = quant.quantize_sb256(w)
    nsb = k // 256
    wg = w.astype(np.float64).reshape(n, nsb, 8, 32)
    sc, mc = quant.unpack_sub(r["sub"])
    d = r["d"].astype(np.float64)
    dm = r["dmin"].astype(np.float64)
    # the nibble layout itself is pinned bit by bit in test_nibble_layout_bitwise
    q = quant.unpack_nibbles(r["qs"]).astype(np.int64).reshape(n, nsb, 8, 32)
    for i in range(n):
        for b in range(nsb):
            hi = wg[i, b].max(-1)
            lo = np.minimum(0.0, wg[i, b].min(-1))
            s = (hi - lo) / 15.0
            # superblock scales: nearest fp16 of the fp64 quantities
            assert int(codecs.f16_bits(r["d"][i, b])) == _nearest_f16_exact(Fraction(float(s.max()) / 63.0))
            assert int(codecs.f16_bits(r["dmin"][i, b])) == _nearest_f16_exact(Fraction(float((-lo).max()) / 63.0))
            for j in range(8):
                for arr, base, target in ((sc, d[i, b], s[j]), (mc, dm[i, b], -lo[j])):
                    if base == 0:
                        assert arr[i, b, j] == 0
                        continue
                    dist = [abs(Fraction(float(target)) - Fraction(float(base)) * c) for c in range(64)]
                    m = min(dist)
                    best = [c for c in range(64) if dist[c] == m]
                    want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                    assert arr[i, b, j] == want
                S = d[i, b] * sc[i, b, j]
                M = dm[i, b] * mc[i, b, j]
                for t in range(32):
                    if S == 0:
                        assert q[i, b, j, t] == 0
                        continue
                    x = Fraction(float(wg[i, b, j, t]))
                    dist = [abs(x - (Fraction(float(S)) * c - Fraction(float(M)))) for c in range(16)]
                    m = min(dist)
                    best = [c for c in range(16) if dist[c] == m]
                    want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                    assert q[i, b, j, t] == want


def test_sb256_brute_force():
    check_sb_brute(seed=21)


# --------------------------------------------------------------------------
# exact round trips of representable weights
# --------------------------------------------------------------------------


def check_sym_roundtrip(bits, group, seed, n=32):
    g = np.random.default_rng(seed)
    Q = (1 << (bits - 1)) - 1
    k = 4 * group
    ng = k // group
    # fp16 scales: normal range, random mantissa
    s16 = (2.0 ** g.integers(-12, 6, (n, ng)) * (1 + g.integers(0, 1024, (n, ng)) / 1024)).astype(np.float16)
    q = g.integers(-Q, Q + 1, (n, k))
    qg = q.reshape(n, ng, group)
    pos = g.integers(0, group, (n, ng))
    sign = np.where(g.random((n, ng)) < 0.5, -Q, Q)
    np.put_along_axis(qg, pos[..., None], sign[..., None], axis=2)
    q = qg.reshape(n, k)
    w64 = (qg * s16.astype(np.float64)[..., None]).reshape(n, k)
    w = w64.astype(np.float32)
    assert np.array_equal(w.astype(np.float64), w64)
    r = quant.quantize_sym(w, bits, group)
    assert np.array_equal(codecs.f16_bits(r["scales"]), codecs.f16_bits(s16))
    assert np.array_equal(r["q"].astype(np.int64), q)
    assert np.array_equal(quant.dequant_sym(r["codes"], r["scales"], bits, group, r.get("hi")), w64)


@pytest.mark.parametrize("bits,group", SYM_CASES)
def test_sym_roundtrip(bits, group):
    check_sym_roundtrip(bits, group, seed=bits + group)


def check_sb_roundtrip(seed, n=16, k=512):
    g = np.random.default_rng(seed)
    nsb = k // 256
    e = g.integers(-10, -6, (n, nsb))
    d16 = (2.0 ** e * (1 + g.integers(0, 1024, (n, nsb)) / 1024)).astype(np.float16)
    m16 = (2.0 ** e * (1 + g.integers(0, 1024, (n, nsb)) / 1024)).astype(np.float16)
    sc = g.integers(1, 64, (n, nsb, 8))
    mc = g.integers(0, 64, (n, nsb, 8))
    sc[:, :, 0] = 63
    mc[:, :, 1] = 63
    q = g.integers(0, 16, (n, nsb, 8, 32))
    q[..., 0] = 0
    q[..., 1] = 15
    S = d16.astype(np.float64)[..., None] * sc
    M = m16.astype(np.float64)[..., None] * mc
    w64 = (S[..., None] * q - M[..., None]).reshape(n, k)
    w = w64.astype(np.float32)
    assert np.array_equal(w.astype(np.float64), w64), "construction not exact in fp32"
    r = quant.quantize_sb256(w)
    assert np.array_equal(codecs.f16_bits(r["d"]), codecs.f16_bits(d16))
    assert np.array_equal(codecs.f16_bits(r["dmin"]), codecs.f16_bits(m16))
    assert np.array_equal(r["sc"].astype(np.int64), sc)
    assert np.array_equal(r["mc"].astype(np.int64), mc)
    assert np.array_equal(r["q"].astype(np.int64), q.reshape(n, k))
    assert np.array_equal(quant.dequant_sb256(r["qs"], r["d"], r["dmin"], r["sub"]), w64)


def test_sb256_zero_offsets_and_ranges_are_positive_zero():
    # a superblock with no negative weight has every group offset 0 and a
    # superblock of signed zeros has every range 0: d and dmin are magnitudes,
    # so they store +0 (0x0000), and all sub-codes and codes are 0
    w = np.zeros((3, 256), np.float32)
    g = np.random.default_rng(4)
    w[0] = np.abs(g.standard_normal(256)).astype(np.float32) + 0.25   # all positive
    w[1] = -0.0                                                       # signed zeros
    w[2, :32] = 0.0                                                   # one constant group
    w[2, 32:] = np.abs(g.standard_normal(224)).astype(np.float32)
    r = quant.quantize_sb256(w)
    assert codecs.f16_bits(r["dmin"][0, 0]) == 0x0000
    assert codecs.f16_bits(r["d"][1, 0]) == 0x0000 and codecs.f16_bits(r["dmin"][1, 0]) == 0x0000
    assert codecs.f16_bits(r["dmin"][2, 0]) == 0x0000
    assert not r["mc"].any()
    assert not r["q"][1].any() and not r["sc"][1].any()


def test_sb256_roundtrip():
    check_sb_roundtrip(seed=4)


def check_rows_roundtrip(kind, seed, n=24, k=64):
    g = np.random.default_rng(seed)
    # scales with <= 16 significant bits so code * scale is exact in fp32
    s = (2.0 ** g.integers(-20, 0, n) * (1 + g.integers(0, 2 ** 15, n) / 2 ** 15)).astype(np.float32)
    if kind == "fp8":
        codes = g.integers(0, 256, (n, k)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x01          # no NaN
        codes[:, 0] = np.where(g.random(n) < 0.5, 0x7E, 0xFE)
        vals = codecs.e4m3_decode(codes)
    else:
        codes = g.integers(-127, 128, (n, k)).astype(np.int8)
        codes[:, 0] = np.where(g.random(n) < 0.5, 127, -127)
        vals = codes.astype(np.float64)
    w64 = vals * s.astype(np.float64)[:, None]
    w = w64.astype(np.float32)
    assert np.array_equal(w.astype(np.float64), w64)
    r = quant.quantize_rows(w, kind)
    assert np.array_equal(r["scales"], s)
    assert np.array_equal(r["codes"].view(np.uint8), codes.view(np.uint8))


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_rows_roundtrip(kind):
    check_rows_roundtrip(kind, seed=11)


# --------------------------------------------------------------------------
# ranges and error bounds
# --------------------------------------------------------------------------


def check_ranges_and_bounds(seed):
    w = _adversarial_weights(32, 512, seed)
    for bits in (4, 8):
        for group in (16, 32, 64):
            r = quant.quantize_sym(w, bits, group)
            Q = (1 << (bits - 1)) - 1
            if bits == 4:
                u = np.concatenate([r["codes"] & 0xF, r["codes"] >> 4])
                assert u.min() >= 1 and u.max() <= 15
            assert np.abs(r["q"].astype(np.int64)).max() <= Q
            s = np.repeat(r["scales"].astype(np.float64), group, axis=1)
            what = quant.dequant_sym(r["codes"], r["scales"], bits, group)
            err = np.abs(w.astype(np.float64) - what)
            a = np.repeat(np.abs(w.astype(np.float64)).reshape(32, -1, group).max(-1), group, axis=1)
            slack = np.maximum(a - Q * s, 0.0)        # clamp at the range edge
            zero = s == 0
            assert np.all(err[~zero] <= s[~zero] / 2 + slack[~zero])
            assert np.all(what[zero] == 0)
    r = quant.quantize_sb256(w)
    assert r["q"].max() <= 15 and r["sc"].max() <= 63 and r["mc"].max() <= 63
    sc, mc = quant.unpack_sub(r["sub"])
    assert sc.max() <= 63 and mc.max() <= 63
    what = quant.dequant_sb256(r["qs"], r["d"], r["dmin"], r["sub"])
    S = np.repeat((r["d"].astype(np.float64)[..., None] * sc).reshape(32, -1), 32, axis=1)
    M = np.repeat((r["dmin"].astype(np.float64)[..., None] * mc).reshape(32, -1), 32, axis=1)
    wd = w.astype(np.float64)
    inside = (wd >= -M) & (wd <= 15 * S - M) & (S > 0)
    assert np.all(np.abs(wd - what)[inside] <= S[inside] / 2 * (1 + 1e-12))
    # outside the representable range the nearest end point is used
    out = ~inside & (S > 0)
    nearest_end = np.minimum(np.abs(wd + M), np.abs(wd - (15 * S - M)))
    assert np.all(np.abs(wd - what)[out] <= nearest_end[out] * (1 + 1e-12) + 1e-300)
    # bound from the format: the representable interval [-M, 15S - M] misses
    # the data interval [lo, hi] by at most 15*d/2 + dmin/2 (6-bit rounding of
    # S and M) plus, where a 6-bit code clamps at 63, 15*63 (resp. 63) times
    # the fp16 rounding error of d (dmin): half an ulp, 2^-11 relative or 2^-25
    # absolute in the subnormal range.  A group whose scale code is 0 spans at
    # most 7.5*d.
    d = np.repeat(np.repeat(r["d"].astype(np.float64), 8, axis=1), 32, axis=1)
    dm = np.repeat(np.repeat(r["dmin"].astype(np.float64), 8, axis=1), 32, axis=1)
    dd = np.maximum(2.0 ** -25, d * 2.0 ** -11)
    ddm = np.maximum(2.0 ** -25, dm * 2.0 ** -11)
    bound = (S / 2 + 7.5 * d + dm / 2 + 945 * dd + 63 * ddm) * (1 + 1e-9)
    assert np.all(np.abs(wd - what) <= bound)
    for kind in ("fp8", "int8"):
        r = quant.quantize_rows(w, kind)
        if kind == "fp8":
            assert not np.any((r["codes"] & 0x7F) == 0x7F)
            v = wd / np.where(r["scales"] == 0, 1, r["scales"]).astype(np.float64)[:, None]
            dec = codecs.e4m3_decode(r["codes"])
            # half a grid step of e4m3fn at |v|: step 2^(e-3), subnormal step 2^-9
            e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
            half = 2.0 ** (e - 3) / 2
            assert np.all(np.abs(v - dec) <= half + np.maximum(np.abs(v) - 448, 0))
        else:
            assert np.abs(r["codes"].astype(np.int64)).max() <= 127


def test_ranges_and_bounds():
    check_ranges_and_bounds(seed=31)


def test_zero_and_nonfinite():
    z = np.zeros((3, 256), dtype=np.float32)
    r = quant.quantize_sym(z, 4, 64)
    assert np.all(r["codes"] == 0x88) and np.all(r["scales"] == 0)
    r = quant.quantize_sb256(z)
    assert np.all(r["qs"] == 0) and np.all(r["d"] == 0) and np.all(r["dmin"] == 0)
    for kind in ("fp8", "int8"):
        r = quant.quantize_rows(z, kind)
        assert np.all(r["scales"] == 0) and np.all(r["codes"].view(np.uint8) == 0)
    bad = np.ones((2, 64), dtype=np.float32)
    bad[1, 3] = np.nan
    with pytest.raises(ValueError):
        quant.quantize_sym(bad, 8, 64)
    bad[1, 3] = np.inf
    with pytest.raises(ValueError):
        quant.quantize_rows(bad, "fp8")
    big = np.full((1, 64), 3e38, dtype=np.float32)   # absmax/7 > 65504
    with pytest.raises(OverflowError):
        quant.quantize_sym(big, 4, 64)


def test_subnormal_fp16_scales_kept():
    # groups small enough that absmax/Q is below the fp16 normal range
    g = np.random.default_rng(2)
    w = (g.standard_normal((4, 64)) * 1e-5).astype(np.float32)
    r = quant.quantize_sym(w, 4, 64)
    s = r["scales"].astype(np.float64)
    assert np.all((s > 0) & (s < 2.0 ** -14))
    check_sym_brute(4, 64, seed=99)


# --------------------------------------------------------------------------
# byte accounting against the model card
# --------------------------------------------------------------------------


def test_checkpoint_bytes_1p5b():
    fig = _golden("page_figures.json")
    layers, c = fig["rwkv7_sizes"]["1.5B"]
    vocab = 65536
    # bytes per weight of w4g64 from the oracle's own buffers on a real row
    r = quant.quantize_sym(np.ones((1, 2048), dtype=np.float32), 4, 64)
    bpw = (r["codes"].nbytes + r["scales"].nbytes) / 2048
    assert bpw == 0.53125
    quantized = layers * 12 * c * c                     # R,K,V,O + cmix key/value
    fp16_rest = 2 * vocab * c                           # embedding + head
    q_bytes = quantized * bpw + fp16_rest * 2
    f_bytes = (quantized + fp16_rest) * 2
    want_q = fig["checkpoint_1p5b"]["int4_g64_GB"] * 1e9
    want_f = fig["checkpoint_1p5b"]["fp16_GB"] * 1e9
    assert abs(q_bytes - want_q) / want_q < 0.05
    assert abs(f_bytes - want_f) / want_f < 0.05


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# --------------------------------------------------------------------------


def test_mutation_floor_instead_of_rne(monkeypatch):
    monkeypatch.setattr(quant, "_rne", np.floor)
    with pytest.raises(AssertionError):
        check_sym_brute(8, 64, seed=1)
    with pytest.raises(AssertionError):
        check_sb_brute(seed=21)


def test_mutation_int4_range(monkeypatch):
    monkeypatch.setattr(quant, "_qmax", lambda bits: 8 if bits == 4 else 127)
    with pytest.raises(AssertionError):
        check_sym_roundtrip(4, 64, seed=3)


def test_mutation_fp16_double_rounding(monkeypatch):
    def via_f32(v):
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float16)
    monkeypatch.setattr(codecs, "f16_encode", via_f32)
    # the codec pin holds a value whose fp32 intermediate lands on an fp16 tie
    with pytest.raises(AssertionError):
        __import__("test_oracle_codecs").test_f16_encode_midpoints_and_neighbours()


def test_nibble_layout_bitwise():
    # bit-by-bit construction of each 32-bit word, independent of the packer:
    # code k = 8w + 2i sits at bits 4i, code k = 8w + 2i + 1 at bits 16 + 4i
    g = np.random.default_rng(17)
    u = g.integers(0, 16, (5, 64)).astype(np.uint8)
    packed = quant.pack_nibbles(u)
    for r in range(5):
        for w in range(8):
            word = 0
            for i in range(4):
                word |= int(u[r, 8 * w + 2 * i]) << (4 * i)
                word |= int(u[r, 8 * w + 2 * i + 1]) << (16 + 4 * i)
            assert packed[r, 4 * w:4 * w + 4].tolist() == [(word >> (8 * b)) & 0xFF for b in range(4)]
    assert np.array_equal(quant.unpack_nibbles(packed), u)


@pytest.mark.parametrize("bits", [5, 6])
def test_hi_plane_bitwise(bits):
    # bit-by-bit construction of each high-plane word, independent of the
    # packer: 6-bit: bits 4i..4i+1 = hi(8w + 2i), 4i+2..4i+3 = hi(8w + 2i + 1);
    # 5-bit: bit i = hi(8w + 2i), bit 4 + i = hi(8w + 2i + 1)
    g = np.random.default_rng(18 + bits)
    u = g.integers(1, 1 << bits, (5, 64)).astype(np.uint8)
    hi = quant.pack_hi(u, bits)
    for r in range(5):
        for w in range(8):
            word = 0
            for i in range(4):
                he, ho = int(u[r, 8 * w + 2 * i]) >> 4, int(u[r, 8 * w + 2 * i + 1]) >> 4
                if bits == 6:
                    word |= (he << (4 * i)) | (ho << (4 * i + 2))
                else:
                    word |= (he << i) | (ho << (4 + i))
            assert int(hi[r, w]) == word, (r, w)
    assert np.array_equal(quant.unpack_hi(hi, bits, 64), u >> 4)
    full = (quant.unpack_nibbles(quant.pack_nibbles(u & 0xF)) | (quant.unpack_hi(hi, bits, 64) << 4))
    assert np.array_equal(full, u)


def test_bf16_encoder_against_torch():
    # a library's float32 -> bfloat16 conversion (round to nearest, ties to
    # even, overflow to infinity) on random magnitudes, midpoints and edges
    import torch
    g = np.random.default_rng(5)
    v = (g.standard_normal(100000) * 10.0 ** g.uniform(-44, 38, 100000)).astype(np.float32)
    top = g.integers(0, 0x7F7F, 20000).astype(np.uint32) << 16
    mids = (top | 0x8000).view(np.float32)                        # exact ties
    near = ((top | 0x8000) + g.choice([-1, 1], 20000).astype(np.uint32)).view(np.float32)
    edges = np.float32([0.0, -0.0, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 3.3895314e38])
    v = np.concatenate([v, mids, -mids, near, edges])
    v = v[np.isfinite(v)]
    mine = codecs.bf16_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(codecs.bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_bf16_quantize_overflow_and_nonfinite():
    with pytest.raises(OverflowError):
        quant.quantize_bf16(np.float32([[3.4e38]]))
    with pytest.raises(ValueError):
        quant.quantize_bf16(np.float32([[np.nan]]))
    r = quant.quantize_bf16(np.float32([[1.0, -2.5, 3.3895314e38]]))
    assert r["codes"].tolist() == [[0x3F80, 0xC020, 0x7F7F]]


def test_mutation_hi_plane_parity(monkeypatch):
    real = quant.pack_hi

    def swapped(u, bits):
        u = np.asarray(u, dtype=np.uint8)
        v = u.copy()
        v[:, 0::2], v[:, 1::2] = u[:, 1::2], u[:, 0::2]   # even / odd exchanged
        return real(v, bits)
    monkeypatch.setattr(quant, "pack_hi", swapped)
    with pytest.raises(AssertionError):
        test_sym_hand_examples_5_6_bits()


def test_mutation_nibble_order(monkeypatch):
    def naive(q, bits):
        u = (np.asarray(q).astype(np.int16) + 8).astype(np.uint8)
        return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(quant, "pack_sym", naive)
    with pytest.raises(AssertionError):
        test_sym_hand_examples("sym_int4_g16", 4)


def test_mutation_sb_offset_not_clamped(monkeypatch):
    monkeypatch.setattr(quant, "_group_low", lambda wd: np.min(wd, axis=3))
    with pytest.raises(AssertionError):
        check_ranges_and_bounds(seed=31)


def test_mutation_fp8_no_saturation(monkeypatch):
    real = codecs.e4m3_encode

    def nonsat(v):
        c = real(v)
        v = np.asarray(v)
        return np.where(np.abs(v) >= 464, (c & 0x80) | 0x7F, c).astype(np.uint8)
    monkeypatch.setattr(codecs, "e4m3_encode", nonsat)
    with pytest.raises(AssertionError):
        test_e4m3_hand = __import__("test_oracle_codecs").test_e4m3_hand_cases
        test_e4m3_hand()
