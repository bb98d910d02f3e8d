"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: quantized codes, scales, mins and sub-codes byte-equal to the oracle;
integer accumulators bit-exact; fp16 outputs within |y - y_ref| <= 2e-3*B +
1e-3 per element and relative L2 <= 1e-3 (oracle.ref.compare), where y_ref
and B = |x| |W_hat|^T are fp64.  Inputs come from gemm_rwkv_amd.synth or
small adversarial generators here; expected values come only from oracle/.
"""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import synth
from gpu_helpers import (Guarded, dev_bytes, dev_f16, dev_f32, host, oracle_buffers,
                         qweight_from_oracle, random_parts, rows_of, say)
from oracle import codecs, quant, ref

pytestmark = pytest.mark.gpu

SYM = [(quant.W4_SYM, 64), (quant.W4_SYM, 32), (quant.W4_SYM, 16),
       (quant.W8_SYM, 64), (quant.W8_SYM, 32), (quant.W8_SYM, 16)]
ALL_SMALL_M = SYM + [(quant.W4_ASYM_SB256, 32), (quant.F16, 0)]


def _weights(n, k, seed, kind="normal"):
    g = np.random.default_rng(seed)
    if kind == "normal":
        return (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    # adversarial: per-row magnitudes over many decades, zero/constant groups, outliers
    w = g.standard_normal((n, k)) * 10.0 ** g.uniform(-7, 3, (n, 1))
    w = w.astype(np.float32)
    if n > 4 and k >= 64:
        w[0, :64] = 0
        w[1, :32] = 0.37
        w[2, :32] = -1.25
        w[3, 7] = 3e3
        w[4, 32:64] = -0.0
    return w


def _quantize_gpu(w, fmt, group):
    n, k = w.shape
    say("quantize", fmt, group, n, k)
    return rq.quantize(dev_f32(w), fmt, group)


def _compare_buffers(qw, fmt, parts, what=""):
    got = qw.buffers()
    want = oracle_buffers(fmt, parts)
    for name, arr in want.items():
        g = host(got[name], np.uint8)
        wb = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
        if not np.array_equal(g, wb):
            bad = np.nonzero(g != wb)[0]
            raise AssertionError("%s %s: %d bytes differ, first at %d (got %d want %d)"
                                 % (what, name, len(bad), bad[0], g[bad[0]], wb[bad[0]]))


# --------------------------------------------------------------------------
# quantizers: byte-exact
# --------------------------------------------------------------------------

QUANT_CASES = [(f, g) for f, g in SYM] + [(quant.W4_ASYM_SB256, 32), (quant.FP8_E4M3_CH, 0),
                                         (quant.I8_CH, 0), (quant.F16, 0)]


@pytest.mark.parametrize("fmt,group", QUANT_CASES)
@pytest.mark.parametrize("n,k,kind", [(7, 256, "normal"), (65, 512, "adversarial"),
                                      (200, 1024, "normal"), (33, 2560, "adversarial")])
def test_quantize_bytes_exact(fmt, group, n, k, kind):
    w = _weights(n, k, seed=n * 7 + k, kind=kind)
    if fmt == quant.F16:
        w = np.clip(w, -60000, 60000)
    parts = quant.quantize(w, fmt, group)
    qw = _quantize_gpu(w, fmt, group)
    torch.cuda.synchronize()
    _compare_buffers(qw, fmt, parts, "fmt %d g %d" % (fmt, group))


def test_quantize_subnormal_superblock_scales():
    # cmix-value-like rows: K = 10240 with N(0, 1/K) weights gives fp16
    # superblock scales below the normal range
    w = _weights(16, 10240, seed=3)
    parts = quant.quantize_sb256(w)
    assert np.any(parts["d"].astype(np.float64) < 2.0 ** -14)
    qw = _quantize_gpu(w, quant.W4_ASYM_SB256, 32)
    _compare_buffers(qw, quant.W4_ASYM_SB256, parts)


def test_quantize_signed_zero_superblocks():
    # superblocks without negative weights, or of signed zeros: d and dmin
    # are stored as +0 on both sides
    g = np.random.default_rng(4)
    w = np.zeros((4, 512), np.float32)
    w[0] = np.abs(g.standard_normal(512)).astype(np.float32) + 0.25
    w[1] = -0.0
    w[2, :256] = -0.0
    w[2, 256:] = g.standard_normal(256).astype(np.float32)
    w[3, :32] = 0.0
    w[3, 32:] = np.abs(g.standard_normal(480)).astype(np.float32)
    parts = quant.quantize_sb256(w)
    qw = _quantize_gpu(w, quant.W4_ASYM_SB256, 32)
    _compare_buffers(qw, quant.W4_ASYM_SB256, parts)
    # and the symmetric formats on signed zeros
    for fmt, group in ((quant.W4_SYM, 32), (quant.W8_SYM, 64)):
        parts = quant.quantize(w, fmt, group)
        _compare_buffers(_quantize_gpu(w, fmt, group), fmt, parts)


def test_quantize_errors():
    w = _weights(8, 128, seed=1)
    w[3, 5] = np.nan
    with pytest.raises(rq.RqError) as e:
        _quantize_gpu(w, quant.W4_SYM, 64)
    assert e.value.status == rq.RQ_ERR_NONFINITE
    w = np.full((2, 64), 3e38, dtype=np.float32)
    with pytest.raises(rq.RqError) as e:
        _quantize_gpu(w, quant.W4_SYM, 64)
    assert e.value.status == rq.RQ_ERR_RANGE


def test_quantize_act_bytes_exact():
    g = np.random.default_rng(9)
    # one-pass kernel: 256, 512 and 1024 threads per row, one or two blocks of
    # 8 per thread (ragged last pass at K = 12304); the looping kernel beyond
    # 2048 blocks (K = 16400)
    for m, k, ldx in [(1, 768, 768), (5, 4096, 4104), (64, 16384, 16384), (3, 16, 16), (7, 8192, 8200),
                      (4, 12304, 12304), (3, 16400, 16408), (2, 2064, 2064)]:
        x = (g.standard_normal((m, ldx)) * 10.0 ** g.uniform(-3, 2, (m, 1))).astype(np.float16)
        x[0, :4] = [0, -0.0, 65504, -1e-7]
        for fmt, kind in ((quant.FP8_E4M3_CH, "fp8"), (quant.I8_CH, "int8")):
            say("quantize_act", m, k, ldx, kind)
            xd = dev_f16(x)
            xq = Guarded(m * k)
            sx = Guarded(4 * m)
            rq.rq_quantize_act(xd, m, k, ldx, fmt, xq.ptr(), sx.ptr())
            want = quant.quantize_rows(x[:, :k], kind)
            assert np.array_equal(host(xq.t, np.uint8), want["codes"].reshape(-1).view(np.uint8))
            assert np.array_equal(host(sx.t, np.float32), want["scales"])
            xq.check_guards()
            sx.check_guards()
    # all-zero row
    x = np.zeros((2, 32), np.float16)
    xq = Guarded(64)
    sx = Guarded(8)
    rq.rq_quantize_act(dev_f16(x), 2, 32, 32, quant.FP8_E4M3_CH, xq.ptr(), sx.ptr())
    assert not host(xq.t, np.uint8).any() and not host(sx.t, np.float32).any()


# --------------------------------------------------------------------------
# weight-streaming products, small shapes with ragged tails
# --------------------------------------------------------------------------


def _run_small_m(qw, x, m, ldx, n):
    xd = dev_f16(x)
    ldy = n + (3 if n % 2 else 0)
    y = Guarded(2 * m * ldy)
    say("small_m", qw.format, qw.group, "m", m, "n", n, "k", qw.k, "ldx", ldx)
    if m == 1 and ldx == qw.k:
        rq.GEMV_ENTRY[(qw.format, qw.group)](xd, qw, y.ptr())
        ldy = n
    else:
        rq.rq_gemm_small_m(xd, m, ldx, qw, y.ptr(), ldy)
    torch.cuda.synchronize()
    y.check_guards()
    out = host(y.t, np.float16)[: m * ldy].reshape(m, ldy)[:, :n]
    return out


@pytest.mark.parametrize("fmt,group", ALL_SMALL_M)
@pytest.mark.parametrize("n,k", [(1, 256), (7, 512), (65, 768), (160, 2048)])
@pytest.mark.parametrize("m", [1, 2, 5, 16, 17, 32])
def test_small_m_parity(fmt, group, n, k, m):
    w = _weights(n, k, seed=n + k + m)
    parts = quant.quantize(w, fmt, group)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    ldx = k + 8
    g = np.random.default_rng(m * 1000 + n)
    x = g.standard_normal((m, ldx)).astype(np.float16)
    y = _run_small_m(qw, x, m, ldx, n)
    y_ref, b = ref.weight_only_ref(x[:, :k], fmt, parts, group)
    ok, info = ref.compare(y, y_ref, b)
    assert ok, info
    if m == 1:
        y1 = _run_small_m(qw, x[:, :k].copy(), 1, k, n)      # the rq_gemv_* entry point
        ok, info = ref.compare(y1, y_ref, b)
        assert ok, info


@pytest.mark.parametrize("fmt,group", SYM + [(quant.W4_ASYM_SB256, 32)])
def test_integer_special_case_exact(fmt, group):
    """Codes with a +-Q entry per group have scale 1 (symmetric), or d = dmin = 1
    (superblocks), so every product and partial sum is an integer below 2^24:
    the output must equal the integer matrix product exactly."""
    g = np.random.default_rng(group)
    # k bounded so that |y| <= 2048 (exact in fp16) for |x| <= 1
    n, m = 48, 8
    k = 256 if fmt == quant.W4_ASYM_SB256 else 128
    if fmt == quant.W4_ASYM_SB256:
        q = g.integers(0, 16, (n, k))
        nsb = k // 256
        parts = {"qs": quant.pack_nibbles(q),
                 "d": np.ones((n, nsb), np.float16), "dmin": np.ones((n, nsb), np.float16),
                 "sub": quant.pack_sub(np.ones((n, nsb, 8), np.uint8), np.full((n, nsb, 8), 8, np.uint8))}
        wint = q - 8
    else:
        Q = 7 if fmt == quant.W4_SYM else 127
        q = g.integers(-min(Q, 3), min(Q, 3) + 1, (n, k))
        q[:, ::group] = np.where(g.random((n, k // group)) < 0.5, -Q, Q)
        parts = quant.quantize(q.astype(np.float32), fmt, group)
        wint = q
    x = g.integers(-1, 2, (m, k)).astype(np.float16)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    y = _run_small_m(qw, x, m, k, n)
    exact = x.astype(np.int64) @ wint.astype(np.int64).T
    assert np.abs(exact).max() <= 2048
    assert np.array_equal(y.astype(np.float64), exact.astype(np.float64))


@pytest.mark.parametrize("fmt,group", [(quant.W4_SYM, 64), (quant.W4_ASYM_SB256, 32), (quant.W8_SYM, 16)])
def test_power_of_two_scaling_and_determinism(fmt, group):
    n, k, m = 96, 1024, 4
    w = _weights(n, k, seed=5)
    parts = quant.quantize(w, fmt, group)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    x = np.random.default_rng(2).standard_normal((m, k)).astype(np.float16)
    y1 = _run_small_m(qw, x, m, k, n)
    y2 = _run_small_m(qw, x, m, k, n)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    y4 = _run_small_m(qw, (x.astype(np.float32) * 4).astype(np.float16), m, k, n)
    assert np.array_equal((y1.astype(np.float32) * 4).astype(np.float16).view(np.uint16), y4.view(np.uint16))


@pytest.mark.parametrize("fmt,group,n,k,m", [
    # shapes whose launch splits K across workgroups and/or groups 2-4 row
    # tiles per workgroup (sharing one activation slice), with ragged tiles
    (quant.W4_SYM, 64, 8192, 2048, 8),      # 2 tiles per workgroup, K unsplit
    (quant.W4_SYM, 64, 2048, 2048, 32),     # unsplit with a 136 KB activation slice in LDS
    (quant.W8_SYM, 32, 2048, 2048, 24),     # the same for int8
    (quant.W4_SYM, 64, 2048, 8192, 32),     # K in 8 slices, 4 tiles per workgroup
    (quant.W4_SYM, 64, 1000, 4096, 32),     # ragged row tiles, split K
    (quant.W4_SYM, 32, 2048, 8192, 1),      # K in 2 slices
    (quant.W8_SYM, 32, 3000, 4096, 20),
    (quant.W8_SYM, 16, 520, 2048, 3),
    (quant.W4_ASYM_SB256, 32, 2560, 10240, 16),
    (quant.F16, 0, 1100, 4096, 32),
])
def test_split_k_and_tile_groups(fmt, group, n, k, m):
    w = _weights(n, k, seed=n + m)
    parts = quant.quantize(w, fmt, group)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    x = synth.act_channel_1202(m, k) if k > 1202 else np.random.default_rng(m).standard_normal((m, k)).astype(np.float16)
    y1 = _run_small_m(qw, x, m, k, n)
    y_ref, b = ref.weight_only_ref(x, fmt, parts, group)
    ok, info = ref.compare(y1, y_ref, b)
    assert ok, info
    # a second call, and a call on another stream with the same workspace,
    # give the same bits
    y2 = _run_small_m(qw, x, m, k, n)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y3 = _run_small_m(qw, x, m, k, n)
    assert np.array_equal(y1.view(np.uint16), y3.view(np.uint16))


def test_fused_rkv_ragged_split():
    """Fused R/K/V at m = 32 on ragged 2000-row matrices: the launch groups row
    tiles and splits K; the last group of each matrix has a tile past its end."""
    k, m = 2048, 32
    ns = [2000, 2000, 1984]
    ws = [_weights(n, k, seed=10 + i) for i, n in enumerate(ns)]
    parts = [quant.quantize(w, quant.W4_SYM, 64) for w in ws]
    qws = [qweight_from_oracle(quant.W4_SYM, 64, p, n, k) for p, n in zip(parts, ns)]
    x = synth.act_channel_1202(m, k)
    ldy = 2008
    ys = [Guarded(2 * m * ldy) for _ in range(3)]
    say("fused_rkv ragged split")
    xd = dev_f16(x)
    rq.rq_fused_rkv(xd, xd, xd, m, k, *qws, *[y.ptr() for y in ys], ldy)
    torch.cuda.synchronize()
    for y, p, n in zip(ys, parts, ns):
        y.check_guards()
        out = host(y.t, np.float16).reshape(m, ldy)[:, :n]
        y_ref, b = ref.weight_only_ref(x, quant.W4_SYM, p, 64)
        ok, info = ref.compare(out, y_ref, b)
        assert ok, info


def test_empty_and_degenerate():
    parts = quant.quantize(np.zeros((16, 64), np.float32), quant.W4_SYM, 64)
    qw = qweight_from_oracle(quant.W4_SYM, 64, parts, 16, 64)
    x = np.ones((3, 64), np.float16)
    y = _run_small_m(qw, x, 3, 64, 16)
    assert not np.any(y)
    y = Guarded(64)
    rq.rq_gemm_small_m(dev_f16(x), 0, 64, qw, y.ptr(), 16)   # m = 0
    torch.cuda.synchronize()
    y.check_guards()


# --------------------------------------------------------------------------
# fused R/K/V
# --------------------------------------------------------------------------


def test_fused_rkv_768_single_call():
    """Width-768 fused R/K/V (RWKV-7 0.1B): int8 symmetric group 64, one call."""
    ws, x = synth.fused_rkv_768()
    parts = [quant.quantize(w, quant.W8_SYM, 64) for w in ws]
    qws = [_quantize_gpu(w, quant.W8_SYM, 64) for w in ws]
    for qw, p in zip(qws, parts):
        _compare_buffers(qw, quant.W8_SYM, p)
    xd = dev_f16(x)
    ys = [Guarded(768 * 2) for _ in range(3)]
    say("fused_rkv 768")
    rq.rq_fused_rkv(xd, xd, xd, 1, 768, *qws, *[y.ptr() for y in ys], 768)
    torch.cuda.synchronize()
    outs = []
    for y, p in zip(ys, parts):
        y.check_guards()
        out = host(y.t, np.float16).reshape(1, 768)
        y_ref, b = ref.weight_only_ref(x, quant.W8_SYM, p, 64)
        ok, info = ref.compare(out, y_ref, b)
        assert ok, info
        outs.append(out)
    # three separate calls agree with the oracle too (the fused launch may cut
    # K differently, so the fp32 summation order need not match bit for bit)
    for qw, p in zip(qws, parts):
        sep = _run_small_m(qw, x, 1, 768, 768)
        y_ref, b = ref.weight_only_ref(x, quant.W8_SYM, p, 64)
        ok, info = ref.compare(sep, y_ref, b)
        assert ok, info


@pytest.mark.parametrize("fmt,group,m", [(quant.W4_SYM, 64, 8), (quant.W4_ASYM_SB256, 32, 3),
                                         (quant.W8_SYM, 32, 32)])
def test_fused_rkv_distinct_inputs(fmt, group, m):
    k = 512
    ns = [64, 80, 33]
    ws = [_weights(n, k, seed=i) for i, n in enumerate(ns)]
    parts = [quant.quantize(w, fmt, group) for w in ws]
    qws = [qweight_from_oracle(fmt, group, p, n, k) for p, n in zip(parts, ns)]
    g = np.random.default_rng(4)
    xs = [g.standard_normal((m, k)).astype(np.float16) for _ in range(3)]
    ldy = 96
    ys = [Guarded(2 * m * ldy) for _ in range(3)]
    say("fused_rkv distinct", fmt, group, m)
    rq.rq_fused_rkv(*[dev_f16(x) for x in xs], m, k, *qws, *[y.ptr() for y in ys], ldy)
    torch.cuda.synchronize()
    for y, x, p, n in zip(ys, xs, parts, ns):
        y.check_guards()
        out = host(y.t, np.float16).reshape(m, ldy)[:, :n]
        y_ref, b = ref.weight_only_ref(x, fmt, p, group)
        ok, info = ref.compare(out, y_ref, b)
        assert ok, info


# --------------------------------------------------------------------------
# W8A8 MFMA GEMMs
# --------------------------------------------------------------------------


def _w8a8(fmt, kind, n, k, m, seed, ldy=None):
    w = _weights(n, k, seed)
    parts = quant.quantize(w, fmt)
    qw = qweight_from_oracle(fmt, 0, parts, n, k)
    x = np.random.default_rng(seed + 1).standard_normal((m, k)).astype(np.float16)
    xq = quant.quantize_rows(x, kind)
    ldy = ldy or n
    y = Guarded(2 * m * ldy)
    say("gemm", kind, "m", m, "n", n, "k", k)
    f = rq.rq_gemm_fp8 if kind == "fp8" else rq.rq_gemm_int8
    f(dev_bytes(xq["codes"]), dev_f32(xq["scales"]), m, qw, y.ptr(), ldy)
    torch.cuda.synchronize()
    y.check_guards()
    out = host(y.t, np.float16).reshape(m, ldy)[:, :n]
    y_ref, b = ref.w8a8_ref(xq["codes"], xq["scales"], kind, fmt, parts)
    return out, y_ref, b, xq, parts, qw


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("n,k,m", [(64, 256, 64), (100, 512, 37), (16, 128, 1), (257, 1024, 130),
                                   # large enough grids for each workgroup tile (64x64, 32x64,
                                   # 32x32), ragged in m and n, odd numbers of k blocks
                                   (4100, 384, 250), (4100, 256, 120), (4000, 640, 100),
                                   # 128x128 tiles on the shared 4-stage ring: ragged m and
                                   # n, 3 k blocks; 2 k blocks; a single k block
                                   (16300, 384, 250), (4100, 256, 1000), (4096, 128, 1024),
                                   # fewer than 256 such tiles: K split over 2 slices (65 k
                                   # blocks: 33 + 32), 4 slices, 2 slices, ragged m and n
                                   (260, 8320, 200), (300, 16384, 129), (600, 8192, 130)])
def test_w8a8_parity(kind, n, k, m):
    fmt = quant.FP8_E4M3_CH if kind == "fp8" else quant.I8_CH
    out, y_ref, b, xq, parts, qw = _w8a8(fmt, kind, n, k, m, seed=n + k + m, ldy=n + 8)
    ok, info = ref.compare(out, y_ref, b)
    assert ok, info
    if kind == "int8":
        acc = Guarded(4 * m * n)
        rq.rq_gemm_int8_acc(dev_bytes(xq["codes"]), m, qw, acc.ptr())
        torch.cuda.synchronize()
        acc.check_guards()
        got = host(acc.t, np.int32).reshape(m, n)
        assert np.array_equal(got.astype(np.int64), ref.int_acc_ref(xq["codes"], parts["codes"]))


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("n,k,m", [(16300, 384, 1000), (16384, 256, 1024), (16000, 128, 1100)])
def test_w8a8_large_tiles(kind, n, k, m):
    """256 x 256 tiles (256 or more of them fill the compute units on their
    own): ragged m and n (1000 = 3 x 256 + 232 rows, 16300 = 63 x 256 + 172
    columns), exact multiples, a single k block.  Sampled output columns,
    the last ones included, against the oracle; int8 accumulators bit-exact."""
    fmt = quant.FP8_E4M3_CH if kind == "fp8" else quant.I8_CH
    w = _weights(n, k, n + k)
    parts = quant.quantize(w, fmt)
    qw = qweight_from_oracle(fmt, 0, parts, n, k)
    x = np.random.default_rng(m + k).standard_normal((m, k)).astype(np.float16)
    xq = quant.quantize_rows(x, kind)
    y = Guarded(2 * m * n)
    say("gemm large tiles", kind, "m", m, "n", n, "k", k)
    f = rq.rq_gemm_fp8 if kind == "fp8" else rq.rq_gemm_int8
    f(dev_bytes(xq["codes"]), dev_f32(xq["scales"]), m, qw, y.ptr(), n)
    torch.cuda.synchronize()
    y.check_guards()
    out = host(y.t, np.float16).reshape(m, n)
    g = np.random.default_rng(n)
    cols = np.concatenate([np.sort(g.choice(n - 40, 88, replace=False)), np.arange(n - 40, n)])
    sub = {name: arr[cols] for name, arr in parts.items()}
    y_ref, b = ref.w8a8_ref(xq["codes"], xq["scales"], kind, fmt, sub)
    ok, info = ref.compare(out[:, cols], y_ref, b)
    assert ok, info
    if kind == "int8":
        acc = Guarded(4 * m * n)
        rq.rq_gemm_int8_acc(dev_bytes(xq["codes"]), m, qw, acc.ptr())
        torch.cuda.synchronize()
        acc.check_guards()
        got = host(acc.t, np.int32).reshape(m, n)[:, cols]
        assert np.array_equal(got.astype(np.int64), ref.int_acc_ref(xq["codes"], parts["codes"][cols]))


def test_fp8_integer_operands_exact():
    """Integer-valued e4m3fn operands with unit scales: the fp32 MFMA sum is
    exact whatever its order, and checks that the matrix core reads OCP e4m3fn."""
    g = np.random.default_rng(0)
    ints = np.array([0.0, 1.0, 2.0, 3.0])
    n, k, m = 64, 128, 32
    x = g.choice(np.concatenate([ints, -ints]), (m, k))
    w = g.choice(np.concatenate([ints, -ints]), (n, k))
    xq = codecs.e4m3_encode(x)
    wq = codecs.e4m3_encode(w)
    qw = rq.QWeight(quant.FP8_E4M3_CH, 0, n, k, dev_bytes(wq), dev_f32(np.ones(n, np.float32)))
    y = Guarded(2 * m * n)
    rq.rq_gemm_fp8(dev_bytes(xq), dev_f32(np.ones(m, np.float32)), m, qw, y.ptr(), n)
    torch.cuda.synchronize()
    exact = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.abs(exact).max() < 2048
    assert np.array_equal(host(y.t, np.float16).reshape(m, n).astype(np.float64), exact.astype(np.float64))


@pytest.mark.parametrize("fmt,group", [(quant.W4_SYM, 64), (quant.W4_SYM, 32), (quant.W4_ASYM_SB256, 32),
                                       (quant.W6_SYM, 64), (quant.W5_SYM, 32)])
@pytest.mark.parametrize("n,k", [(3100, 2560), (4000, 4096), (3580, 8192), (200, 4096)])
def test_streamed_activation_chunks(fmt, group, n, k):
    """M > 16 with an activation slice too large for one workgroup's LDS and
    192..256 row tiles: each wave streams its own chunks through a private
    double buffer (K = 2560 leaves the last wave with a ragged chunk range;
    rows >= M read zeros; n = 3100 and 3580 end in a partial tile).  The
    200-row case takes the split plan."""
    w = _weights(n, k, seed=n * 5 + k)
    parts = quant.quantize(w, fmt, group)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    ldx = k + 16
    for m in (17, 24, 32):
        g = np.random.default_rng(m + k)
        x = g.standard_normal((m, ldx)).astype(np.float16)
        y = _run_small_m(qw, x, m, ldx, n)
        y_ref, b = ref.weight_only_ref(x[:, :k], fmt, parts, group)
        ok, info = ref.compare(y, y_ref, b)
        assert ok, (m, info)


@pytest.mark.parametrize("fmt,group,k", [(quant.W4_SYM, 64, 128 * 131), (quant.W4_SYM, 32, 128 * 131),
                                         (quant.W8_SYM, 64, 64 * 133), (quant.W8_SYM, 16, 64 * 133),
                                         (quant.F16, 0, 32 * 131), (quant.BF16, 0, 32 * 131)])
@pytest.mark.parametrize("m", [1, 2])
def test_sixteen_chunk_waves(fmt, group, k, m):
    """With 128 or more row tiles and 128 or more chunks in the slice, M <= 2
    gives waves of sixteen chunks that keep a window of eight code loads in
    flight and issue the rest while they compute.  K is 131 or 133 chunks, so
    the last wave of a tile holds 3 or 5 valid chunks and 13 or 11 past the
    end (their codes read zero, their scales are dropped); n = 2085 ends in a
    partial tile.  Codes and scales are seeded random bytes (inputs); the
    oracle multiplies sampled rows."""
    n = 2085
    g = np.random.default_rng(k + m)
    full = random_parts(fmt, group, n, k, g)
    qw = qweight_from_oracle(fmt, group, full, n, k)
    ldx = k + 8
    x = g.standard_normal((m, ldx)).astype(np.float16)
    y = _run_small_m(qw, x, m, ldx, n)
    rows = np.concatenate([np.sort(g.choice(n - 5, 24, replace=False)), np.arange(n - 5, n)])
    y_ref, b = ref.weight_only_ref(x[:, :k], fmt, rows_of(full, rows), group)
    ok, info = ref.compare(y[:, rows], y_ref, b)
    assert ok, info


@pytest.mark.parametrize("fmt,group,k", [(quant.W4_SYM, 64, 16000), (quant.W4_SYM, 32, 16384),
                                         (quant.W4_ASYM_SB256, 32, 16128), (quant.W6_SYM, 32, 16000),
                                         (quant.W5_SYM, 64, 16384)])
def test_streamed_one_tile(fmt, group, k):
    """M = 4..8 with an activation slice too large for one workgroup's LDS
    and 192..256 row tiles: each wave streams its chunks (16 rows, rows >= M
    read zeros) through a private double buffer.  K = 16000 and 16128 leave
    the last wave with 5 or 6 of its 8 chunks; n = 3100 ends in a partial
    tile.  Codes are seeded random bytes; the oracle multiplies sampled
    rows."""
    n = 3100
    g = np.random.default_rng(k + group)
    parts = random_parts(fmt, group, n, k, g)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    rows = np.concatenate([np.sort(g.choice(n - 4, 28, replace=False)), np.arange(n - 4, n)])
    for m in (4, 7, 8):
        ldx = k + 8 * m
        x = g.standard_normal((m, ldx)).astype(np.float16)
        y = _run_small_m(qw, x, m, ldx, n)
        y_ref, b = ref.weight_only_ref(x[:, :k], fmt, rows_of(parts, rows), group)
        ok, info = ref.compare(y[:, rows], y_ref, b)
        assert ok, (m, info)


@pytest.mark.parametrize("n,k", [(9, 64 * 13), (33, 64 * 5), (300, 64 * 129), (2085, 64 * 133)])
@pytest.mark.parametrize("m", [1, 2, 5, 17])
def test_int8_g64_odd_groups_per_row(n, k, m):
    """int8 with group 64 is the one format whose rows can hold an odd number
    of fp16 scales, so a row's scales end in the middle of a dword; the last
    row's last scale shares its dword with the bytes after the buffer (this
    once lost that scale to the buffer range check)."""
    w = _weights(n, k, seed=n + k)
    parts = quant.quantize(w, quant.W8_SYM, 64)
    qw = qweight_from_oracle(quant.W8_SYM, 64, parts, n, k)
    g = np.random.default_rng(n * 7 + m)
    x = g.standard_normal((m, k)).astype(np.float16)
    y = _run_small_m(qw, x, m, k, n)
    y_ref, b = ref.weight_only_ref(x, quant.W8_SYM, parts, 64)
    ok, info = ref.compare(y, y_ref, b)
    assert ok, info
    # the last row's error is fp16 output rounding only; one dropped chunk of
    # 64 k would move it by about |y| / sqrt(chunks)
    assert np.all(np.abs(y[:, -1] - y_ref[:, -1]) <= 4e-3 * np.abs(y_ref[:, -1]) + 2e-3)
