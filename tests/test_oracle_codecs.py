"""Pins for the oracle's number codecs (CPU only).

fp16: exhaustive decode against the binary16 closed form, and every midpoint
between neighbouring values (ties to even, subnormals, overflow).
e4m3fn: exhaustive decode against torch's float8_e4m3fn, brute-force nearest
search for the encoder, hand-derived cases, and torch's RNE conversion on
inputs inside the finite range.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16_closed_form(bits):
    s = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0x1F:
        return s * math.inf if m == 0 else math.nan
    if e == 0:
        return s * m * 2.0 ** -24
    return s * (1024 + m) * 2.0 ** (e - 25)


def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = codecs.f16_from_bits(bits).astype(np.float64)
    want = np.array([_f16_closed_form(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # -0.0 keeps its sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_f16_encode_midpoints_and_neighbours():
    # all non-negative finite binary16 values in increasing order
    vals = np.array([_f16_closed_form(b) for b in range(0x7C00)])
    assert np.all(np.diff(vals) > 0)
    mids = (vals[:-1] + vals[1:]) / 2.0          # exact in fp64
    enc = codecs.f16_bits(codecs.f16_encode(mids)).astype(np.int64)
    lo_code = np.arange(0x7C00 - 1)
    even_pick = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)
    assert np.array_equal(enc, even_pick)
    up = codecs.f16_bits(codecs.f16_encode(np.nextafter(mids, np.inf))).astype(np.int64)
    dn = codecs.f16_bits(codecs.f16_encode(np.nextafter(mids, -np.inf))).astype(np.int64)
    assert np.array_equal(up, lo_code + 1)
    assert np.array_equal(dn, lo_code)
    # exact values are fixed points, negative side mirrors
    assert np.array_equal(codecs.f16_bits(codecs.f16_encode(vals)), np.arange(0x7C00))
    neg = codecs.f16_bits(codecs.f16_encode(-vals[1:])).astype(np.int64)
    assert np.array_equal(neg, np.arange(1, 0x7C00) | 0x8000)
    # overflow: the midpoint between 65504 and 2^16 rounds to infinity
    assert codecs.f16_encode(65519.99).item() == 65504.0
    assert math.isinf(codecs.f16_encode(65520.0).item())
    # the double-rounding trap: fp64 -> fp32 -> fp16 would give 1.0 here
    assert codecs.f16_encode(1 + 2.0 ** -11 + 2.0 ** -40).item() == 1 + 2.0 ** -10


def test_e4m3_decode_matches_torch_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.E4M3_TABLE
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(t[~nan], ours[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ours[~nan]))


def test_e4m3_hand_cases():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["e4m3fn"]["cases"]
    for v, code in cases:
        got = int(codecs.e4m3_encode(np.array([v]))[0])
        assert got == int(code, 16), (v, hex(got), code)


def _brute_e4m3(v):
    """Nearest finite code with the sign of v; ties to even code; saturating."""
    best = None
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    for c in range(0x7F):  # magnitudes 0x00..0x7E
        d = abs(a - codecs.E4M3_TABLE[c])
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | sign


def test_e4m3_encode_brute_force():
    g = np.random.default_rng(12)
    v = np.concatenate([
        g.standard_normal(1500) * 10.0 ** g.uniform(-4, 3, 1500),
        (codecs.E4M3_TABLE[:0x7E] + codecs.E4M3_TABLE[1:0x7F]) / 2.0,   # every midpoint
        -(codecs.E4M3_TABLE[:0x7E] + codecs.E4M3_TABLE[1:0x7F]) / 2.0,
        [448.0, 449.0, 463.9, 464.0, 1e6, -1e6, 0.0, -0.0, 1e-300, -1e-300],
    ])
    got = codecs.e4m3_encode(v)
    want = np.array([_brute_e4m3(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn is RNE but does not saturate: compare
    # only inside [-448, 448] where the two definitions coincide.
    g = np.random.default_rng(5)
    v = (g.standard_normal(200000) * 10.0 ** g.uniform(-4, 2.6, 200000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode(v.astype(np.float64)), t)


def test_e4m3_rejects_nonfinite():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([np.nan]))
