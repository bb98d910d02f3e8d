"""Round-to-nearest quantizers producing the canonical byte layouts (oracle).

Test infrastructure only: tests, the smoke check and bench's cpu_baseline leg
may call this module; the GPU library never does.

All arithmetic that decides a code or a scale is a fixed sequence of IEEE fp64
operations followed by a single rounding to the target grid, exactly as
written below.  "RNE" is round-half-to-even (``numpy.rint``).

Formats (a weight matrix is W[N][K]: N output rows, K contiguous inputs, and the
product is ``y[m][n] = sum_k x[m][k] * W[n][k]``):

W8_SYM / W4_SYM, group G in {16, 32, 64} along K
    Symmetric round-to-nearest with one fp16 scale per (row, group).  Pages:
    "RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang" (summary; "Format & loading":
    group-wise GROUP=64 symmetric int4, ``.qweight`` + ``.scale``, and the int8
    w8g64 tier in the accuracy warning) and the rwkv-quant news article
    ("Dois presets e seis tamanhos": 8-bit symmetric projections, group 16).
    For b bits the code range is symmetric about zero, Q = 2**(b-1) - 1
    (127 for int8, 7 for int4) and ``s = fp16(absmax / Q)``.  The int4 reading
    (codes -7..7, -8 unused) extends the int8 rule; the pages do not print it
    ("parity unpinned by the pages": pinned by the exact round-trip tests).
    int8 codes: two's complement int8 [N][K].
    int4 codes: offset binary u = q + 8 in 1..15, eight per little-endian
    32-bit word (see pack_nibbles): uint8 [N][K/2].  Scales: fp16 [N][K/G].

W4_ASYM_SB256
    Asymmetric 4-bit codes in superblocks of 256 = 8 groups of 32 (news
    article, "Dois presets e seis tamanhos": 4-bit asymmetric superblock layout,
    group 32).  Per group j: lo_j = min(0, min w), hi_j = max w,
    s_j = (hi_j - lo_j) / 15.  Per superblock: d = fp16(max_j s_j / 63),
    dmin = fp16(max_j(-lo_j) / 63); 6-bit sub-codes
    sc_j = clamp(RNE(s_j / d), 0, 63), mc_j = clamp(RNE(-lo_j / dmin), 0, 63);
    effective S_j = d * sc_j, M_j = dmin * mc_j; codes
    q = clamp(RNE((w + M_j) / S_j), 0, 15); w_hat = S_j * q - M_j.
    The article chooses scale and offset by an activation-weighted search; this
    format uses plain RTN for them ("parity unpinned by the pages").
    Storage: qs uint8 [N][K/2] (nibbles as pack_nibbles), d fp16 [N][K/256],
    dmin fp16 [N][K/256], sub uint8 [N][K/256][12] = a little-endian 96-bit
    stream with sc_j at bit 6j and mc_j at bit 48 + 6j.

W6_SYM / W5_SYM, group G in {32, 64}
    The 6- and 5-bit widths of the presets (news article, "Dois presets e seis
    tamanhos": channel-mix weights at 6 bits in one preset; channel-mix key and
    head at 5 bits in the other).  The article gives their widths only; the
    reading here is the symmetric group rule above at b = 6 / 5 (Q = 31 / 15,
    s = fp16(absmax / Q)), with codes stored in two planes so that the 4-bit
    machinery reads the low plane unchanged.  Offset binary u = q + 2**(b-1)
    (1..63 or 1..31).  Low plane: u & 15 as pack_nibbles, uint8 [N][K/2].
    High plane (pack_hi): for every 8-k word w, the high bits u >> 4 of
    k = 8w + 2i (even) and 8w + 2i + 1 (odd), i = 0..3:
      6-bit: one little-endian uint16 per word, nibble i = hi(even) | hi(odd) << 2
             -> uint16 [N][K/8];
      5-bit: one byte per word, bit i = hi(even), bit 4 + i = hi(odd)
             -> uint8 [N][K/8].
    Scales fp16 [N][K/G].  ("parity unpinned by the pages"; pinned by brute
    force, exact round trips and a hand-derived layout fixture.)

BF16
    Plain bfloat16 weights (news article, "Onde o 2.9B quebra": the layer-0
    output projection kept in bf16): the nearest bfloat16 (8-bit significand,
    fp32's exponent range) to each fp32 weight, ties to even; uint16 bits
    [N][K].  A weight that rounds past the largest finite bfloat16 raises
    OverflowError.

FP8_E4M3_CH / I8_CH
    Per-output-channel scale in fp32, FP8 e4m3fn or int8 codes ("RWKV-7
    Quantization Toolkit", Key Design: FP8 weights on FP8 tensor cores, INT8
    weights through int8 x int8 dot products).  s_n = fp32(absmax_n / 448)
    (fp8) or fp32(absmax_n / 127) (int8); codes e4m3fn_rne_sat(w / s_n) or
    clamp(RNE(w / s_n), -127, 127).

Per-token activation quantization uses the same per-row rule on x[M][K]
(both operands of the int8 x int8 and fp8 x fp8 products are quantized).

Zero scales (all-zero group, or a scale that rounds to zero) give all-zero
codes (0x00 for fp8).  Non-finite inputs raise ValueError; a scale that
overflows its storage type raises OverflowError.
"""

import numpy as np

from . import codecs

W8_SYM = 1
W4_SYM = 2
W4_ASYM_SB256 = 3
FP8_E4M3_CH = 4
I8_CH = 5
F16 = 6
W5_SYM = 7
W6_SYM = 8
BF16 = 9

SYM_BITS = {W8_SYM: 8, W6_SYM: 6, W5_SYM: 5, W4_SYM: 4}

SB = 256          # superblock length
SB_GROUP = 32     # group length inside a superblock
SB_NGROUPS = SB // SB_GROUP


def _check_finite(a):
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input")


def _rne(v):
    return np.rint(v)


def _group_low(wd):
    """Lower end of each 32-group's range: min(0, min w) (zero stays reachable)."""
    return np.minimum(0.0, np.min(wd, axis=3))


def _qmax(bits):
    """Largest code magnitude of a b-bit symmetric code: 2**(b-1) - 1."""
    return (1 << (bits - 1)) - 1


# --------------------------------------------------------------------------
# symmetric group RTN
# --------------------------------------------------------------------------


def quantize_sym(w, bits, group):
    """Symmetric group RTN of fp32 W[N][K]; returns dict(codes, scales, q).

    ``q`` is the unpacked int code array [N][K] (int8), ``codes`` the stored
    layout, ``scales`` fp16 [N][K/group].
    """
    w = np.asarray(w, dtype=np.float32)
    _check_finite(w)
    n, k = w.shape
    check_sym_shape(bits, group, k)
    qmax = _qmax(bits)
    wd = w.astype(np.float64).reshape(n, k // group, group)
    absmax = np.max(np.abs(wd), axis=2)
    s16 = codecs.f16_encode(absmax / float(qmax))
    if not np.all(np.isfinite(s16)):
        raise OverflowError("fp16 scale overflow")
    s = s16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(_rne(wd / s), -qmax, qmax)
    q = np.where(s == 0.0, 0.0, q).astype(np.int8).reshape(n, k)
    return sym_parts(q, s16, bits)


def check_sym_shape(bits, group, k):
    """Raise ValueError unless (bits, group, K) is a symmetric group format."""
    groups = (16, 32, 64) if bits in (4, 8) else (32, 64)
    if bits not in (4, 5, 6, 8) or group not in groups or k % group or k % 8:
        raise ValueError("unsupported bits/group/shape")


def sym_parts(q, s16, bits):
    """The stored buffers of symmetric codes q [N][K] with fp16 scales s16:
    dict(codes, scales, q), plus ``hi`` (the high plane) at 5 and 6 bits."""
    out = {"codes": pack_sym(q, bits), "scales": s16, "q": q}
    if bits in (5, 6):
        out["hi"] = pack_hi((np.asarray(q).astype(np.int16) + (1 << (bits - 1))).astype(np.uint8), bits)
    return out


def pack_nibbles(u):
    """4-bit values u[N][K] (0..15, K % 8 == 0) -> uint8 [N][K/2].

    The library's int4 layout (the pages give none): each run of 8
    consecutive k is one little-endian 32-bit word; bits 4i..4i+3 hold
    k = 2i (even k in the low half-word) and bits 16+4i..16+4i+3 hold
    k = 2i+1.  As bytes: [u0|u2<<4, u4|u6<<4, u1|u3<<4, u5|u7<<4].
    """
    u = np.asarray(u, dtype=np.uint8)
    n, k = u.shape
    w = u.reshape(n, k // 8, 8)
    out = np.empty((n, k // 8, 4), dtype=np.uint8)
    out[..., 0] = w[..., 0] | (w[..., 2] << 4)
    out[..., 1] = w[..., 4] | (w[..., 6] << 4)
    out[..., 2] = w[..., 1] | (w[..., 3] << 4)
    out[..., 3] = w[..., 5] | (w[..., 7] << 4)
    return out.reshape(n, k // 2)


def unpack_nibbles(c):
    """uint8 [N][K/2] in the pack_nibbles layout -> 4-bit values [N][K] (uint8)."""
    c = np.asarray(c, dtype=np.uint8)
    n, kh = c.shape
    b = c.reshape(n, kh // 4, 4)
    u = np.empty((n, kh // 4, 8), dtype=np.uint8)
    u[..., 0] = b[..., 0] & 0xF
    u[..., 2] = b[..., 0] >> 4
    u[..., 4] = b[..., 1] & 0xF
    u[..., 6] = b[..., 1] >> 4
    u[..., 1] = b[..., 2] & 0xF
    u[..., 3] = b[..., 2] >> 4
    u[..., 5] = b[..., 3] & 0xF
    u[..., 7] = b[..., 3] >> 4
    return u.reshape(n, 2 * kh)


def pack_sym(q, bits):
    """Unpacked int codes [N][K] -> stored code layout: int8, or the low-nibble
    plane of the offset codes u = q + 2**(b-1) (all of u at 4 bits)."""
    q = np.asarray(q)
    if bits == 8:
        return q.astype(np.int8)
    u = (q.astype(np.int16) + (1 << (bits - 1))).astype(np.uint8)
    return pack_nibbles(u & 0xF)


def pack_hi(u, bits):
    """High plane of 5/6-bit offset codes u [N][K] (see W6_SYM / W5_SYM)."""
    u = np.asarray(u, dtype=np.uint8)
    n, k = u.shape
    h = (u >> 4).reshape(n, k // 8, 8).astype(np.uint16)
    if bits == 6:
        out = np.zeros((n, k // 8), dtype=np.uint16)
        for i in range(4):
            out |= (h[..., 2 * i] | (h[..., 2 * i + 1] << 2)) << (4 * i)
        return out
    if bits == 5:
        out = np.zeros((n, k // 8), dtype=np.uint16)
        for i in range(4):
            out |= (h[..., 2 * i] << i) | (h[..., 2 * i + 1] << (4 + i))
        return out.astype(np.uint8)
    raise ValueError("high plane exists at 5 and 6 bits only")


def unpack_hi(hi, bits, k):
    """High plane -> the high bits u >> 4 [N][K] (uint8)."""
    hi = np.asarray(hi)
    n = hi.shape[0]
    hv = hi.reshape(n, k // 8).astype(np.uint16)
    h = np.empty((n, k // 8, 8), dtype=np.uint8)
    for i in range(4):
        if bits == 6:
            h[..., 2 * i] = (hv >> (4 * i)) & 3
            h[..., 2 * i + 1] = (hv >> (4 * i + 2)) & 3
        else:
            h[..., 2 * i] = (hv >> i) & 1
            h[..., 2 * i + 1] = (hv >> (4 + i)) & 1
    return h.reshape(n, k)


def unpack_sym(codes, bits, hi=None):
    """Stored layout -> unpacked int codes [N][K] (int8)."""
    if bits == 8:
        return np.asarray(codes).view(np.int8)
    u = unpack_nibbles(codes).astype(np.int16)
    if bits in (5, 6):
        u = u | (unpack_hi(hi, bits, u.shape[1]).astype(np.int16) << 4)
    return (u - (1 << (bits - 1))).astype(np.int8)


def dequant_sym(codes, scales, bits, group, hi=None):
    q = unpack_sym(codes, bits, hi).astype(np.float64)
    n, k = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    return (q.reshape(n, k // group, group) * s[:, :, None]).reshape(n, k)


# --------------------------------------------------------------------------
# asymmetric 4-bit superblocks
# --------------------------------------------------------------------------


def quantize_sb256(w):
    """Asymmetric superblock RTN of fp32 W[N][K] (K % 256 == 0).

    Returns dict(qs, d, dmin, sub, q, sc, mc).
    """
    w = np.asarray(w, dtype=np.float32)
    _check_finite(w)
    n, k = w.shape
    if k % SB:
        raise ValueError("K must be a multiple of 256")
    nsb = k // SB
    wd = w.astype(np.float64).reshape(n, nsb, SB_NGROUPS, SB_GROUP)
    hi = np.max(wd, axis=3)
    lo = _group_low(wd)
    # fp64 group scale and offset.  Both are magnitudes (the offset is stored
    # as an unsigned code that is subtracted), so a zero is +0: a range or an
    # offset of zero must not become -0 and store 0x8000 as d or dmin.
    s = (hi - lo) / 15.0
    s = np.where(s == 0.0, 0.0, s)
    neglo = 0.0 - lo
    return sb256_from_group_params(wd, s, neglo)


def sb256_from_group_params(wd, s, neglo):
    """The superblock step of the SB256 format from each group's fp64 scale s
    and offset magnitude -lo (both [N][nsb][8]), for weights wd
    [N][nsb][8][32] (fp64): two-level fp16 d / dmin with 6-bit sub-codes, then
    the codes against the effective S_j and M_j."""
    n, nsb = wd.shape[0], wd.shape[1]
    k = nsb * SB
    d16 = codecs.f16_encode(np.max(s, axis=2) / 63.0)
    m16 = codecs.f16_encode(np.max(neglo, axis=2) / 63.0)
    if not (np.all(np.isfinite(d16)) and np.all(np.isfinite(m16))):
        raise OverflowError("fp16 superblock scale overflow")
    d = d16.astype(np.float64)[:, :, None]
    dm = m16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.clip(_rne(s / d), 0, 63)
        mc = np.clip(_rne(neglo / dm), 0, 63)
    sc = np.where(d == 0.0, 0.0, sc)
    mc = np.where(dm == 0.0, 0.0, mc)
    S = d * sc                                 # exact: 11-bit x 6-bit
    M = dm * mc
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(_rne((wd + M[..., None]) / S[..., None]), 0, 15)
    q = np.where(S[..., None] == 0.0, 0.0, q)
    q = q.astype(np.uint8).reshape(n, k)
    sc = sc.astype(np.uint8)
    mc = mc.astype(np.uint8)
    qs = pack_nibbles(q)
    return {"qs": qs, "d": d16, "dmin": m16, "sub": pack_sub(sc, mc),
            "q": q, "sc": sc, "mc": mc}


def pack_sub(sc, mc):
    """6-bit codes sc, mc [N][nsb][8] -> uint8 [N][nsb][12] bit stream.

    Bit i of the 96-bit little-endian stream is bit (i % 8) of byte i // 8;
    sc_j occupies bits 6j .. 6j+5 and mc_j bits 48+6j .. 48+6j+5.
    """
    sc = np.asarray(sc, dtype=np.uint64)
    mc = np.asarray(mc, dtype=np.uint64)
    lo48 = np.zeros(sc.shape[:-1], dtype=np.uint64)
    hi48 = np.zeros(sc.shape[:-1], dtype=np.uint64)
    for j in range(SB_NGROUPS):
        lo48 |= sc[..., j] << np.uint64(6 * j)
        hi48 |= mc[..., j] << np.uint64(6 * j)
    out = np.empty(sc.shape[:-1] + (12,), dtype=np.uint8)
    for b in range(6):
        out[..., b] = (lo48 >> np.uint64(8 * b)) & np.uint64(0xFF)
        out[..., 6 + b] = (hi48 >> np.uint64(8 * b)) & np.uint64(0xFF)
    return out


def unpack_sub(sub):
    """uint8 [N][nsb][12] -> (sc, mc) uint8 [N][nsb][8]."""
    sub = np.asarray(sub, dtype=np.uint8).astype(np.uint64)
    lo48 = np.zeros(sub.shape[:-1], dtype=np.uint64)
    hi48 = np.zeros(sub.shape[:-1], dtype=np.uint64)
    for b in range(6):
        lo48 |= sub[..., b] << np.uint64(8 * b)
        hi48 |= sub[..., 6 + b] << np.uint64(8 * b)
    sc = np.stack([(lo48 >> np.uint64(6 * j)) & np.uint64(63) for j in range(8)], -1)
    mc = np.stack([(hi48 >> np.uint64(6 * j)) & np.uint64(63) for j in range(8)], -1)
    return sc.astype(np.uint8), mc.astype(np.uint8)


def dequant_sb256(qs, d, dmin, sub):
    q = unpack_nibbles(qs).astype(np.float64)
    n, k = q.shape
    sc, mc = unpack_sub(sub)
    dd = np.asarray(d, dtype=np.float16).astype(np.float64)[:, :, None]
    dm = np.asarray(dmin, dtype=np.float16).astype(np.float64)[:, :, None]
    S = dd * sc.astype(np.float64)
    M = dm * mc.astype(np.float64)
    q = q.reshape(n, k // SB, SB_NGROUPS, SB_GROUP)
    return (S[..., None] * q - M[..., None]).reshape(n, k)


# --------------------------------------------------------------------------
# per-row (per-output-channel weights / per-token activations) fp8 and int8
# --------------------------------------------------------------------------


def quantize_rows(a, kind):
    """Per-row scale quantization of a[R][K] (fp32 weights or fp16 activations).

    kind 'fp8': s = fp32(absmax/448), codes e4m3fn (uint8).
    kind 'int8': s = fp32(absmax/127), codes int8 in -127..127.
    Returns dict(codes, scales) with fp32 scales [R].
    """
    a = np.asarray(a)
    _check_finite(a)
    ad = a.astype(np.float64)
    absmax = np.max(np.abs(ad), axis=1)
    if kind == "fp8":
        s32 = (absmax / codecs.E4M3_MAX).astype(np.float32)
    elif kind == "int8":
        s32 = (absmax / 127.0).astype(np.float32)
    else:
        raise ValueError(kind)
    if not np.all(np.isfinite(s32)):
        raise OverflowError("fp32 scale overflow")
    s = s32.astype(np.float64)[:, None]
    zero = s == 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = np.where(zero, 0.0, ad / np.where(zero, 1.0, s))
    if kind == "fp8":
        codes = codecs.e4m3_encode(quo)
        codes = np.where(zero, np.uint8(0), codes).astype(np.uint8)
    else:
        codes = np.clip(_rne(quo), -127, 127).astype(np.int8)
    return {"codes": codes, "scales": s32}


def dequant_rows(codes, scales, kind):
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]
    if kind == "fp8":
        return codecs.e4m3_decode(codes) * s
    return np.asarray(codes).view(np.int8).astype(np.float64) * s


# --------------------------------------------------------------------------
# uniform front door
# --------------------------------------------------------------------------


def quantize_bf16(w):
    """fp32 W -> bfloat16 bits (uint16), nearest with ties to even."""
    w = np.asarray(w, dtype=np.float32)
    _check_finite(w)
    b = codecs.bf16_encode(w.astype(np.float64))
    if np.any((b & 0x7FFF) == 0x7F80):
        raise OverflowError("bfloat16 overflow")
    return {"codes": b}


def quantize(w, fmt, group=0):
    """Quantize fp32 W[N][K] into format ``fmt``; returns a dict of buffers."""
    if fmt in SYM_BITS:
        return quantize_sym(w, SYM_BITS[fmt], group)
    if fmt == W4_ASYM_SB256:
        return quantize_sb256(w)
    if fmt == FP8_E4M3_CH:
        return quantize_rows(np.asarray(w, dtype=np.float32), "fp8")
    if fmt == I8_CH:
        return quantize_rows(np.asarray(w, dtype=np.float32), "int8")
    if fmt == F16:
        return {"codes": np.asarray(w, dtype=np.float16)}
    if fmt == BF16:
        return quantize_bf16(w)
    raise ValueError("unknown format")


def dequant(fmt, parts, group=0):
    """Dequantize a dict of buffers (as returned by ``quantize``) to fp64 W_hat."""
    if fmt in SYM_BITS:
        return dequant_sym(parts["codes"], parts["scales"], SYM_BITS[fmt], group, parts.get("hi"))
    if fmt == W4_ASYM_SB256:
        return dequant_sb256(parts["qs"], parts["d"], parts["dmin"], parts["sub"])
    if fmt == FP8_E4M3_CH:
        return dequant_rows(parts["codes"], parts["scales"], "fp8")
    if fmt == I8_CH:
        return dequant_rows(parts["codes"], parts["scales"], "int8")
    if fmt == F16:
        return np.asarray(parts["codes"], dtype=np.float16).astype(np.float64)
    if fmt == BF16:
        return codecs.bf16_decode(parts["codes"])
    raise ValueError("unknown format")
