"""Number codecs used by the quantized formats (oracle; test infrastructure only).

fp16
    IEEE-754 binary16.  Encoding from fp64 is numpy's ``float64 -> float16``
    conversion, which is one round-to-nearest-even step with gradual underflow
    (subnormals kept, no flush to zero) and overflow to +-inf.  The pins in
    ``tests/test_oracle_codecs.py`` check that claim exhaustively rather than
    trusting it.

e4m3fn
    The OCP 8-bit floating point "E4M3" encoding used by FP8 tensor-core GEMMs
    ("RWKV-7 Quantization Toolkit", Key Design: FP8 weights go through FP8
    tensor cores).  Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 holds subnormals ``m * 2**-9``; the two codes with all
    exponent and mantissa bits set (0x7F, 0xFF) are NaN; there is no infinity, so
    the largest finite magnitude is ``1.75 * 2**8 = 448``.  The encoder here
    rounds to the nearest representable value with ties to the even code and
    saturates magnitudes above 448 to 448; the sign of zero is kept.
"""

import numpy as np

# --------------------------------------------------------------------------
# fp16
# --------------------------------------------------------------------------


def f16_encode(v):
    """fp64 values -> fp16 (numpy float16 array), one RNE rounding."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def f16_bits(h):
    """fp16 array -> its uint16 bit patterns."""
    return np.ascontiguousarray(np.asarray(h, dtype=np.float16)).view(np.uint16)


def f16_from_bits(bits):
    """uint16 bit patterns -> fp16 array."""
    return np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.float16)


# --------------------------------------------------------------------------
# bfloat16
# --------------------------------------------------------------------------
# bfloat16 keeps fp32's sign and 8-bit exponent and the top 7 stored mantissa
# bits.  Every finite fp32 value lies between two consecutive bfloat16 values
# (its top 16 bits, and the next one up in magnitude); the encoder picks the
# nearer, and the one with an even last mantissa bit on a tie.  Distances are
# exact in fp64.  A value that rounds up past the largest finite bfloat16 gives
# infinity (0x7F80 / 0xFF80).


def bf16_decode(bits):
    """uint16 bfloat16 patterns -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_encode(v):
    """Values exactly representable in fp32 -> nearest bfloat16 bits (uint16)."""
    f = np.asarray(v, dtype=np.float64)
    f32 = f.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), f, equal_nan=True):
        raise ValueError("bf16_encode takes values representable in fp32")
    bits = f32.view(np.uint32)
    lo = (bits >> 16).astype(np.uint16)              # truncation toward zero
    hi = (lo + 1).astype(np.uint16)                  # next magnitude up
    a = np.abs(f)
    dlo = a - np.abs(bf16_decode(lo))
    # past the largest finite value the next magnitude is 2**128 (the
    # rounding is done as if the exponent were unbounded; picking it overflows)
    hv = np.where((hi & 0x7FFF) == 0x7F80, 2.0 ** 128, np.abs(bf16_decode(hi)))
    dhi = hv - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


# --------------------------------------------------------------------------
# e4m3fn
# --------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def _e4m3_value(code):
    """Value of one e4m3fn code from the definition (NaN for 0x7F/0xFF)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite values, indexed by code 0x00..0x7E; strictly increasing.
_POS_VALUES = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes):
    """uint8 e4m3fn codes -> fp64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """fp64 values -> uint8 e4m3fn codes: nearest value, ties to even, saturating.

    Implemented as a search over the table of representable magnitudes (not by
    bit manipulation): for each |v| the two neighbouring table entries are the
    candidates, the closer one wins and an exact tie goes to the code whose
    mantissa LSB (= code LSB) is 0.  Magnitudes >= 448 give 448.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(v)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    vlo = _POS_VALUES[lo]
    vhi = _POS_VALUES[hi]
    dlo = a - vlo
    dhi = vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    # exact hits (a == vhi) have dhi == 0 and are picked by the first clause
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    neg = np.signbit(v)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)
