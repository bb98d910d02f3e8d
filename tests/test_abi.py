"""CPU tests of the C ABI: the library loads, exports every declared symbol,
reports sizes, and rejects bad arguments before touching the GPU.

No call here reaches a kernel launch: every call either fails validation or
has an empty extent (m == 0 / n == 0), both of which return before any HIP
runtime call.  Fake device addresses are plain integers.
"""

import json
import os
import re

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rq.h")

A = 0x7f0000000000          # a 16-byte aligned fake device address
B = 0x7f0010000000
C = 0x7f0020000000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(rq.EXPORTS)
    L = rq.lib()
    for name in names:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    L = rq.lib()
    assert L.rq_abi_version() == 5
    assert rq.rq_workspace_bytes() == 64 << 20
    for st in range(-10, 1):
        assert rq.status_str(st) and rq.status_str(st) != "unknown status"
    assert rq.status_str(-99) == "unknown status"


def test_qweight_bytes():
    assert rq.rq_qweight_bytes(rq.RQ_W4_SYM, 64, 2048, 2048) == (2048 * 1024, 2048 * 32 * 2, 0, 0)
    assert rq.rq_qweight_bytes(rq.RQ_W8_SYM, 16, 3, 32) == (96, 3 * 2 * 2, 0, 0)
    assert rq.rq_qweight_bytes(rq.RQ_W4_ASYM_SB256, 32, 2560, 10240) == (
        2560 * 5120, 2560 * 40 * 2, 2560 * 40 * 2, 2560 * 40 * 12)
    assert rq.rq_qweight_bytes(rq.RQ_FP8_E4M3_CH, 0, 4096, 16384) == (4096 * 16384, 4096 * 4, 0, 0)
    assert rq.rq_qweight_bytes(rq.RQ_F16, 0, 65536, 4096) == (65536 * 4096 * 2, 0, 0, 0)
    # SB256 is 4.5 bits per weight, w4g64 4.25
    c, s, m, sub = rq.rq_qweight_bytes(rq.RQ_W4_ASYM_SB256, 32, 1, 256)
    assert (c + s + m + sub) * 8 / 256 == 4.5
    # 6 and 5 bits: low plane k/2, fp16 scales, high plane k/4 or k/8 bytes
    assert rq.rq_qweight_bytes(rq.RQ_W6_SYM, 32, 2560, 10240) == (2560 * 5120, 2560 * 320 * 2, 0, 2560 * 2560)
    assert rq.rq_qweight_bytes(rq.RQ_W5_SYM, 64, 3, 256) == (3 * 128, 3 * 4 * 2, 0, 3 * 32)
    assert rq.rq_qweight_bytes(rq.RQ_BF16, 0, 2560, 2560) == (2560 * 2560 * 2, 0, 0, 0)
    c, s, m, sub = rq.rq_qweight_bytes(rq.RQ_W6_SYM, 64, 1, 128)
    assert (c + s + m + sub) * 8 / 128 == 6.25
    c, s, m, sub = rq.rq_qweight_bytes(rq.RQ_W5_SYM, 32, 1, 128)
    assert (c + s + m + sub) * 8 / 128 == 5.5
    for bad in [(rq.RQ_W4_SYM, 48, 4, 96), (10, 0, 4, 64), (rq.RQ_W4_ASYM_SB256, 64, 4, 256),
                (rq.RQ_W6_SYM, 16, 4, 128), (rq.RQ_W5_SYM, 48, 4, 128)]:
        with pytest.raises(rq.RqError) as e:
            rq.rq_qweight_bytes(*bad)
        assert e.value.status == rq.RQ_ERR_FORMAT
    for bad in [(rq.RQ_W4_SYM, 64, 4, 96), (rq.RQ_W4_ASYM_SB256, 32, 4, 128), (rq.RQ_W8_SYM, 16, -1, 16),
                (rq.RQ_W8_SYM, 16, 1, 0), (rq.RQ_F16, 0, 1, 12), (rq.RQ_W8_SYM, 16, 2 ** 31, 16),
                (rq.RQ_W6_SYM, 32, 4, 96), (rq.RQ_W5_SYM, 64, 4, 192), (rq.RQ_BF16, 0, 4, 48)]:
        with pytest.raises(rq.RqError) as e:
            rq.rq_qweight_bytes(*bad)
        assert e.value.status == rq.RQ_ERR_SHAPE


def test_checkpoint_bytes_from_library():
    """1.5B at w4g64 with fp16 embedding and head is ~1.2 GB; all fp16 ~2.9 GB
    (model card summary).  Uses the library's own size helper."""
    with open(os.path.join(ROOT, "tests", "golden", "page_figures.json")) as f:
        fig = json.load(f)
    layers, c = fig["rwkv7_sizes"]["1.5B"]
    q = 0
    f16 = 0
    for n, k in [(c, c)] * 4 + [(4 * c, c), (c, 4 * c)]:
        q += sum(rq.rq_qweight_bytes(rq.RQ_W4_SYM, 64, n, k)) * layers
        f16 += sum(rq.rq_qweight_bytes(rq.RQ_F16, 0, n, k)) * layers
    emb_head = 2 * sum(rq.rq_qweight_bytes(rq.RQ_F16, 0, 65536, c))
    assert abs((q + emb_head) / 1e9 - fig["checkpoint_1p5b"]["int4_g64_GB"]) < 0.05
    assert abs((f16 + emb_head) / 1e9 - fig["checkpoint_1p5b"]["fp16_GB"]) < 0.1


def _w(fmt=rq.RQ_W4_SYM, group=64, n=32, k=128, codes=A, scales=B, mins=None, sub=None):
    return rq.QWeight(fmt, group, n, k, codes, scales, mins, sub)


def _status(fn, *args):
    with pytest.raises(rq.RqError) as e:
        fn(*args)
    return e.value.status


def test_gemv_validation():
    y = C
    assert _status(rq.rq_gemv_w4g64, 0, _w(), y) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(), 0) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(codes=0), y) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(scales=0), y) == rq.RQ_ERR_NULL
    # wrong entry point for the format / group
    assert _status(rq.rq_gemv_w4g32, A + 0x100000, _w(), y) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemv_w8g64, A + 0x100000, _w(), y) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(group=48), y) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemv_w4sb256, A + 0x100000, _w(), y) == rq.RQ_ERR_FORMAT
    # k not a multiple of the group
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(k=96), y) == rq.RQ_ERR_SHAPE
    # misaligned
    assert _status(rq.rq_gemv_w4g64, A + 0x100008, _w(), y) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(codes=A + 4), y) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(), y + 2) == rq.RQ_ERR_ALIGN
    # output overlapping the codes or x
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(), A + 16) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_gemv_w4g64, A + 0x100000, _w(), A + 0x100000) == rq.RQ_ERR_ALIAS
    # SB256 needs mins and sub
    sb = _w(rq.RQ_W4_ASYM_SB256, 32, 8, 256, A, B, None, C + 0x1000)
    assert _status(rq.rq_gemv_w4sb256, A + 0x100000, sb, C) == rq.RQ_ERR_NULL
    # empty output rows: nothing to do
    rq.rq_gemv_w4g64(A + 0x100000, _w(n=0), C)


def test_small_m_and_fused_validation():
    w = _w()
    x = A + 0x200000
    assert _status(rq.rq_gemm_small_m, x, 33, 128, w, C, 32) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_small_m, x, -1, 128, w, C, 32) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_small_m, x, 4, 120, w, C, 32) == rq.RQ_ERR_SHAPE   # ldx < k
    assert _status(rq.rq_gemm_small_m, x, 4, 132, w, C, 32) == rq.RQ_ERR_ALIGN   # ldx % 8
    assert _status(rq.rq_gemm_small_m, x, 4, 128, w, C, 31) == rq.RQ_ERR_SHAPE   # ldy < n
    assert _status(rq.rq_gemm_small_m, x, 4, 128, _w(rq.RQ_FP8_E4M3_CH, 0), C, 32) == rq.RQ_ERR_FORMAT
    rq.rq_gemm_small_m(x, 0, 128, w, C, 32)          # m == 0: no-op
    w2 = _w(codes=A + 0x10000, scales=B + 0x10000)
    w3 = _w(codes=A + 0x20000, scales=B + 0x20000)
    ys = (C, C + 0x1000, C + 0x2000)
    assert _status(rq.rq_fused_rkv, x, x, x, 1, 128, w, w2, _w(rq.RQ_W8_SYM, 64, codes=A + 0x20000),
                   *ys, 32) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_fused_rkv, x, x, x, 1, 128, w, w2, _w(k=256, codes=A + 0x20000),
                   *ys, 32) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_fused_rkv, x, x, x, 1, 128, w, w2, w3, C, C, C + 0x2000, 32) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_fused_rkv, x, x, x, 1, 128, w, w2, w3, C, C + 0x1000, x, 32) == rq.RQ_ERR_ALIAS
    rq.rq_fused_rkv(x, x, x, 0, 128, w, w2, w3, *ys, 32)  # m == 0, shared x: valid no-op


def test_gemm_w4_validation():
    w = _w(rq.RQ_W4_SYM, 64, 32, 256, A, B)
    x, y = C, C + 0x100000
    assert _status(rq.rq_gemm_w4, x, 4, 256, _w(rq.RQ_W8_SYM, 64, 32, 256, A, B), y, 32) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemm_w4, x, 4, 256, _w(rq.RQ_FP8_E4M3_CH, 0, 32, 256, A, B), y, 32) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemm_w4, x, 4, 192, _w(rq.RQ_W4_SYM, 64, 32, 192, A, B), y, 32) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_w4, x, -1, 256, w, y, 32) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_w4, x, 4, 248, w, y, 32) == rq.RQ_ERR_SHAPE     # ldx < k
    assert _status(rq.rq_gemm_w4, x, 4, 260, w, y, 32) == rq.RQ_ERR_ALIGN     # ldx % 8
    assert _status(rq.rq_gemm_w4, x, 4, 256, w, y, 31) == rq.RQ_ERR_SHAPE     # ldy < n
    assert _status(rq.rq_gemm_w4, 0, 4, 256, w, y, 32) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemm_w4, x + 8, 4, 256, w, y, 32) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_gemm_w4, x, 4, 256, w, A + 0x10, 32) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_gemm_w4, x, 4, 256, w, x, 32) == rq.RQ_ERR_ALIAS
    rq.rq_gemm_w4(x, 0, 256, w, y, 32)                   # m == 0: no-op
    rq.rq_gemm_w4(x, 4, 256, _w(rq.RQ_W4_SYM, 64, 0, 256, A, B), y, 32)  # n == 0: no-op


def test_quantize_and_gemm_validation():
    qw = _w(rq.RQ_W4_SYM, 64, 16, 128)
    assert _status(rq.rq_quantize_rtn, 0, qw) == rq.RQ_ERR_NULL
    assert _status(rq.rq_quantize_rtn, A + 4, _w(codes=B, scales=C)) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_quantize_rtn, A, _w(codes=A + 0x100, scales=C)) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_quantize_rtn, A, _w(codes=B, scales=B + 0x10)) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_quantize_rtn, A, _w(rq.RQ_W4_SYM, 64, 16, 100, B, C)) == rq.RQ_ERR_SHAPE
    rq.rq_quantize_rtn(A, _w(n=0, codes=B, scales=C))   # empty: no-op
    f8 = _w(rq.RQ_FP8_E4M3_CH, 0, 64, 256, A, B)
    i8 = _w(rq.RQ_I8_CH, 0, 64, 256, A, B)
    xq, sx, y = C, C + 0x100000, C + 0x200000
    assert _status(rq.rq_gemm_fp8, xq, sx, 4, i8, y, 64) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemm_int8, xq, sx, 4, f8, y, 64) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemm_fp8, xq, sx, 4, _w(rq.RQ_FP8_E4M3_CH, 0, 64, 144, A, B), y, 64) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_fp8, 0, sx, 4, f8, y, 64) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemm_fp8, xq, 0, 4, f8, y, 64) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemm_fp8, xq, sx, 4, f8, y, 63) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_fp8, xq, sx, 4, f8, A, 64) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_gemm_int8, xq, sx, 4, _w(rq.RQ_I8_CH, 0, 8, 131072 + 128, A, B), y, 64) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_int8_acc, xq, 4, i8, 0) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemm_int8_acc, xq, 4, i8, xq) == rq.RQ_ERR_ALIAS
    rq.rq_gemm_fp8(xq, sx, 0, f8, y, 64)                # m == 0: no-op
    assert _status(rq.rq_quantize_act, A, 4, 256, 256, rq.RQ_W4_SYM, B, C) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_quantize_act, A, 4, 136, 136, rq.RQ_FP8_E4M3_CH, B, C) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_quantize_act, A, 4, 256, 256, rq.RQ_FP8_E4M3_CH, 0, C) == rq.RQ_ERR_NULL
    assert _status(rq.rq_quantize_act, A, 4, 256, 256, rq.RQ_FP8_E4M3_CH, A + 0x100, C) == rq.RQ_ERR_ALIAS
    rq.rq_quantize_act(A, 0, 256, 256, rq.RQ_I8_CH, B, C)


# --------------------------------------------------------------------------
# the library's own rounding routines, run on the host, against libraries
# --------------------------------------------------------------------------


def _f16_grid():
    v = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2
    return np.concatenate([v, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                           [65519.99, 65520.0, 1e6, 1e-30, 2.0 ** -25, 2.0 ** -26]])


def test_host_convert_f16_against_numpy():
    v = _f16_grid()
    v = np.concatenate([v, -v])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(rq.rq_host_convert(0, v), want)


def test_host_convert_f32_against_numpy():
    g = np.random.default_rng(0)
    v = g.standard_normal(200000) * 10.0 ** g.uniform(-45, 38, 200000)
    f32 = np.float32
    edges = np.array([np.finfo(f32).tiny, np.finfo(f32).tiny / 2 ** 23, np.finfo(f32).tiny / 2 ** 24,
                      np.finfo(f32).tiny / 2 ** 24 * 1.0000001, 3.4028235e38, 3.4028236e38, 3.5e38])
    v = np.concatenate([v, edges, -edges])
    with np.errstate(over="ignore"):
        want = v.astype(np.float32).view(np.uint32)
    assert np.array_equal(rq.rq_host_convert(1, v), want)


def test_host_convert_e4m3_against_torch():
    g = np.random.default_rng(1)
    v = (g.standard_normal(300000) * 10.0 ** g.uniform(-5, 2.7, 300000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = rq.rq_host_convert(2, v.astype(np.float64))
    assert np.array_equal(got, want)
    # saturation and signed zero (torch does not saturate, so hand values)
    got = rq.rq_host_convert(2, np.array([449.0, 464.0, 1e9, -1e9, -0.0, -1e-30]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80]


def test_quantize_aw_validation():
    qw = _w(rq.RQ_W4_SYM, 64, 16, 128, B, C)
    imp = A + 0x100000
    assert _status(rq.rq_quantize_aw, A, 0, qw) == rq.RQ_ERR_NULL
    assert _status(rq.rq_quantize_aw, 0, imp, qw) == rq.RQ_ERR_NULL
    assert _status(rq.rq_quantize_aw, A, imp, _w(rq.RQ_FP8_E4M3_CH, 0, 16, 128, B, C)) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_quantize_aw, A, imp, _w(rq.RQ_I8_CH, 0, 16, 128, B, C)) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_quantize_aw, A, imp, _w(rq.RQ_F16, 0, 16, 128, B)) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_quantize_aw, A, imp + 4, qw) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_quantize_aw, A + 4, imp, qw) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_quantize_aw, A, B + 0x10, qw) == rq.RQ_ERR_ALIAS      # act_sq inside the codes
    assert _status(rq.rq_quantize_aw, A, C, qw) == rq.RQ_ERR_ALIAS             # act_sq on the scales
    assert _status(rq.rq_quantize_aw, A, imp, _w(rq.RQ_W4_SYM, 64, 16, 100, B, C)) == rq.RQ_ERR_SHAPE
    sb = _w(rq.RQ_W4_ASYM_SB256, 32, 4, 384, B, C, C + 0x1000, C + 0x2000)
    assert _status(rq.rq_quantize_aw, A, imp, sb) == rq.RQ_ERR_SHAPE         # K % 256
    rq.rq_quantize_aw(A, imp, _w(n=0, codes=B, scales=C))                    # empty: no-op


def test_two_plane_and_bf16_validation():
    x, y = C, C + 0x100000
    w6 = _w(rq.RQ_W6_SYM, 32, 32, 256, A, B, None, A + 0x10000)
    assert _status(rq.rq_gemm_small_m, x, 4, 256, _w(rq.RQ_W6_SYM, 32, 32, 256, A, B), y, 32) == rq.RQ_ERR_NULL
    assert _status(rq.rq_gemm_small_m, x, 4, 256, _w(rq.RQ_W5_SYM, 32, 32, 256, A, B, None, A + 0x10008),
                   y, 32) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_gemm_small_m, x, 4, 256, _w(rq.RQ_W6_SYM, 16, 32, 256, A, B, None, A + 0x10000),
                   y, 32) == rq.RQ_ERR_FORMAT
    assert _status(rq.rq_gemm_small_m, x, 4, 256, w6, A + 0x10000, 32) == rq.RQ_ERR_ALIAS  # y on the high plane
    assert _status(rq.rq_quantize_rtn, x, _w(rq.RQ_W6_SYM, 32, 32, 192, A, B, None, A + 0x10000)) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_small_m, x, 4, 48, _w(rq.RQ_BF16, 0, 32, 48, A), y, 32) == rq.RQ_ERR_SHAPE
    assert _status(rq.rq_gemm_w4, x, 4, 256, w6, y, 32) == rq.RQ_ERR_FORMAT
    rq.rq_gemm_small_m(x, 0, 256, w6, y, 32)   # m == 0: no-op


def test_workspace_validation():
    """A workspace must be 16-byte aligned and disjoint from the call's inputs
    and outputs; without one (NULL) any size is ignored."""
    w = _w()
    x = A + 0x200000
    y = C
    W = 0x7f0050000000
    assert _status(rq.rq_gemm_small_m, x, 1, 128, w, y, 32, None, (W + 8, 1 << 20)) == rq.RQ_ERR_ALIGN
    assert _status(rq.rq_gemm_small_m, x, 1, 128, w, y, 32, None, (y - 64, 1 << 20)) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_gemm_small_m, x, 1, 128, w, y, 32, None, (A, 4096)) == rq.RQ_ERR_ALIAS    # codes
    assert _status(rq.rq_gemm_small_m, x, 1, 128, w, y, 32, None, (x - 16, 4096)) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_gemv_w4g64, x, w, y, None, (B, 64)) == rq.RQ_ERR_ALIAS                     # scales
    assert _status(rq.rq_gemm_w4, x, 1, 128, w, y, 32, None, (y, 64)) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_fused_rkv, x, x, x, 1, 128, w, w, w, y, y + 0x1000, y + 0x2000, 32, None,
                   (y + 0x2000, 64)) == rq.RQ_ERR_ALIAS
    f8 = _w(rq.RQ_FP8_E4M3_CH, 0, 32, 128)
    assert _status(rq.rq_gemm_fp8, x, x + 0x10000, 1, f8, y, 32, None, (x, 64)) == rq.RQ_ERR_ALIAS
    assert _status(rq.rq_gemm_int8_acc, x, 1, _w(rq.RQ_I8_CH, 0, 32, 128), y, None, (y + 16, 64)) == rq.RQ_ERR_ALIAS
    # empty extents with a workspace return before any launch
    rq.rq_gemm_small_m(x, 0, 128, w, y, 32, ws=(W, 1 << 20))
    rq.rq_gemm_small_m(x, 1, 128, _w(n=0), y, 32, ws=False)


def test_noalloc_limits():
    """rq_gemm_small_m_noalloc refuses products whose partial sums could
    exceed its 8 MiB scratch, before any device call."""
    x = A + 0x200000
    assert _status(rq.rq_gemm_small_m_noalloc, x, 17, 128, _w(n=4112), C, 4112) == rq.RQ_ERR_SCRATCH
    assert _status(rq.rq_gemm_small_m_noalloc, x, 1, 128, _w(n=8208), C, 8208) == rq.RQ_ERR_SCRATCH
    assert _status(rq.rq_gemm_small_m_noalloc, x, 1, 128, _w(codes=0), C, 32) == rq.RQ_ERR_NULL
    assert rq.lib().rq_gemm_small_m_noalloc(x, 1, 128, None, C, 32, None) == rq.RQ_ERR_NULL
    # within the limit, validation still applies
    assert _status(rq.rq_gemm_small_m_noalloc, x, 33, 128, _w(), C, 32) == rq.RQ_ERR_SHAPE
    rq.rq_gemm_small_m_noalloc(x, 0, 128, _w(n=4096), C, 4096)       # empty: nothing to do


def test_stream_read_validation():
    assert rq.lib().rq_stream_read(None, 16, A, None) == rq.RQ_ERR_NULL
    assert rq.lib().rq_stream_read(A, 16, None, None) == rq.RQ_ERR_NULL
    assert rq.lib().rq_stream_read(A + 8, 16, B, None) == rq.RQ_ERR_ALIGN
    assert rq.lib().rq_stream_read(A, 16, B + 2, None) == rq.RQ_ERR_ALIGN
    assert rq.lib().rq_stream_read(A, 20, B, None) == rq.RQ_ERR_SHAPE
