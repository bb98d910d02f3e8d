"""Parity at the workloads' full sizes, in the launch shapes bench.py times.

Weights are generated on the host from the seeded generators, quantized on
the GPU with rq_quantize_rtn, and used by the same entry points as the
benchmark (rq_fused_rkv, rq_gemm_small_m, rq_gemv_*, rq_quantize_act,
rq_gemm_fp8/int8).  The oracle quantizes only a sample of rows (each row's
codes depend on that row alone), checks their bytes against the GPU's, and
computes the outputs of those rows for every activation row.
"""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import synth
from gpu_helpers import dev_f16, dev_f32, host, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu

SAMPLE = 48  # rows checked per matrix


def _rows(n, seed):
    g = np.random.default_rng(seed)
    pick = g.choice(n, size=min(SAMPLE, n), replace=False)
    return np.sort(np.concatenate([pick, [0, n - 1]]) if n > 2 else pick).astype(np.int64)


def _gpu_weights(w, fmt, group):
    return rq.quantize(dev_f32(w), fmt, group)


def _check_rows_sym(qw, w, rows, fmt, group):
    """Bytes of the sampled rows against the oracle; returns their parts."""
    n, k = w.shape
    bits = 4 if fmt == quant.W4_SYM else 8
    parts = quant.quantize_sym(w[rows], bits, group)
    cb = k // 2 if bits == 4 else k
    codes = host(qw.codes, np.uint8)[: n * cb].reshape(n, cb)[rows]
    scales = host(qw.scales, np.uint16)[: n * (k // group)].reshape(n, k // group)[rows]
    assert np.array_equal(codes, parts["codes"].reshape(len(rows), -1).view(np.uint8)), "codes differ"
    assert np.array_equal(scales, parts["scales"].view(np.uint16)), "scales differ"
    return parts


def _check_rows_sb(qw, w, rows):
    n, k = w.shape
    nsb = k // 256
    parts = quant.quantize_sb256(w[rows])
    got = {
        "qs": host(qw.codes, np.uint8)[: n * k // 2].reshape(n, k // 2)[rows],
        "d": host(qw.scales, np.uint16)[: n * nsb].reshape(n, nsb)[rows],
        "dmin": host(qw.mins, np.uint16)[: n * nsb].reshape(n, nsb)[rows],
        "sub": host(qw.sub, np.uint8)[: n * nsb * 12].reshape(n, nsb, 12)[rows],
    }
    assert np.array_equal(got["qs"], parts["qs"])
    assert np.array_equal(got["d"], parts["d"].view(np.uint16))
    assert np.array_equal(got["dmin"], parts["dmin"].view(np.uint16))
    assert np.array_equal(got["sub"], parts["sub"])
    return parts


def _compare_rows(y, rows, x, fmt, parts, group, what):
    y_ref, b = ref.weight_only_ref(x, fmt, parts, group)
    ok, info = ref.compare(y[:, rows], y_ref, b)
    assert ok, (what, info)


# --------------------------------------------------------------------------
# width 2048 (1.5B) layer, int4 g64, every M from 1 to 32: the benchmark's
# decode (M = 1, 8, 32) and every plan between (two-range tiles up to M = 8,
# streaming tiles, the phased kernel past M = 16, K splits summed in launch)
# --------------------------------------------------------------------------


@pytest.fixture(scope="module")
def layer_2048():
    c = 2048
    mats = {}
    for mat, n, k in synth.layer_shapes(c):
        w = synth.weight(1, 0, mat, n, k)
        mats[mat] = (w, _gpu_weights(w, quant.W4_SYM, 64))
    yield c, mats
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", list(range(1, 33)))
def test_decode_layer_2048(layer_2048, m):
    c, mats = layer_2048
    x = synth.act_channel_1202(m, c)
    x4 = synth.act_normal(m, 4 * c, 1)
    xd, x4d = dev_f16(x), dev_f16(x4)
    say("decode layer 2048 m", m, rq.rq_plan_small_m(mats[synth.MAT_VALUE][1], m, 4 * c))
    ys = {mat: torch.empty(m * n * 2, dtype=torch.uint8, device="cuda") for mat, n, _ in synth.layer_shapes(c)}
    q = {mat: mats[mat][1] for mat in mats}
    rq.rq_fused_rkv(xd, xd, xd, m, c, q[synth.MAT_R], q[synth.MAT_K], q[synth.MAT_V],
                    ys[synth.MAT_R], ys[synth.MAT_K], ys[synth.MAT_V], c)
    rq.rq_gemm_small_m(xd, m, c, q[synth.MAT_O], ys[synth.MAT_O], c)
    rq.rq_gemm_small_m(xd, m, c, q[synth.MAT_KEY], ys[synth.MAT_KEY], 4 * c)
    rq.rq_gemm_small_m(x4d, m, 4 * c, q[synth.MAT_VALUE], ys[synth.MAT_VALUE], c)
    torch.cuda.synchronize()
    for mat, n, k in synth.layer_shapes(c):
        w = mats[mat][0]
        rows = _rows(n, 100 + mat)
        parts = _check_rows_sym(q[mat], w, rows, quant.W4_SYM, 64)
        y = host(ys[mat], np.float16).reshape(m, n)
        _compare_rows(y, rows, x4 if k == 4 * c else x, quant.W4_SYM, parts, 64, synth.MAT_NAMES[mat])


# --------------------------------------------------------------------------
# width 2560 (2.9B): O, cmix key, cmix value as SB256, x with 8 massive channels
# --------------------------------------------------------------------------


@pytest.mark.parametrize("m", [1, 4, 16])
def test_sb256_2560(m):
    c = 2560
    for mat, n, k in [(synth.MAT_O, c, c), (synth.MAT_KEY, 4 * c, c), (synth.MAT_VALUE, c, 4 * c)]:
        w = synth.weight(2, 0, mat, n, k)
        qw = _gpu_weights(w, quant.W4_ASYM_SB256, 32)
        x = synth.act_massive(m, k)
        y = torch.empty(m * n * 2, dtype=torch.uint8, device="cuda")
        say("sb256 2560", synth.MAT_NAMES[mat], "m", m)
        if m == 1:
            rq.rq_gemv_w4sb256(dev_f16(x), qw, y)
        else:
            rq.rq_gemm_small_m(dev_f16(x), m, k, qw, y, n)
        torch.cuda.synchronize()
        rows = _rows(n, 200 + mat)
        parts = _check_rows_sb(qw, w, rows)
        _compare_rows(host(y, np.float16).reshape(m, n), rows, x, quant.W4_ASYM_SB256, parts, 32,
                      synth.MAT_NAMES[mat])


# --------------------------------------------------------------------------
# width 4096 (7.2B) prefill set: fp8 and int8 per channel, M in {64, 256, 1024}
# --------------------------------------------------------------------------


@pytest.fixture(scope="module")
def prefill_4096():
    c = 4096
    ws = {mat: synth.weight(3, 0, mat, n, k) for mat, n, k in synth.layer_shapes(c)}
    q = {}
    for kind, fmt in (("fp8", quant.FP8_E4M3_CH), ("int8", quant.I8_CH)):
        q[kind] = {mat: _gpu_weights(w, fmt, 0) for mat, w in ws.items()}
    yield c, ws, q
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("m", [64, 256, 1024])
def test_prefill_4096(prefill_4096, kind, m):
    c, ws, q = prefill_4096
    fmt = quant.FP8_E4M3_CH if kind == "fp8" else quant.I8_CH
    for mat, n, k in synth.layer_shapes(c):
        x = synth.act_normal(m, k, 3, salt=mat)
        xq = torch.empty(m * k, dtype=torch.uint8, device="cuda")
        sx = torch.empty(m, dtype=torch.float32, device="cuda")
        say("prefill 4096", kind, synth.MAT_NAMES[mat], "m", m)
        rq.rq_quantize_act(dev_f16(x), m, k, k, fmt, xq, sx)
        y = torch.empty(m * n * 2, dtype=torch.uint8, device="cuda")
        f = rq.rq_gemm_fp8 if kind == "fp8" else rq.rq_gemm_int8
        f(xq, sx, m, q[kind][mat], y, n)
        torch.cuda.synchronize()
        # activation rows: sampled bytes; weight rows: sampled bytes
        arows = _rows(m, 300 + mat)
        px = quant.quantize_rows(x[arows], kind)
        assert np.array_equal(host(xq, np.uint8).reshape(m, k)[arows], px["codes"].reshape(len(arows), k).view(np.uint8))
        assert np.array_equal(host(sx, np.float32)[arows], px["scales"])
        rows = _rows(n, 400 + mat)
        pw = quant.quantize_rows(ws[mat][rows], kind)
        qw = q[kind][mat]
        assert np.array_equal(host(qw.codes, np.uint8)[: n * k].reshape(n, k)[rows],
                              pw["codes"].reshape(len(rows), k).view(np.uint8))
        assert np.array_equal(host(qw.scales, np.float32)[:n][rows], pw["scales"])
        y_ref, b = ref.w8a8_ref(px["codes"], px["scales"], kind, fmt, pw)
        got = host(y, np.float16).reshape(m, n)[np.ix_(arows, rows)]
        ok, info = ref.compare(got, y_ref, b)
        assert ok, (kind, synth.MAT_NAMES[mat], m, info)


# --------------------------------------------------------------------------
# width 4096 (7.2B) prefill set on int4 g64 codes (rq_gemm_w4), M in
# {64, 256, 1024}
# --------------------------------------------------------------------------


@pytest.fixture(scope="module")
def prefill_w4_4096():
    c = 4096
    mats = {}
    for mat, n, k in synth.layer_shapes(c):
        w = synth.weight(3, 10, mat, n, k)
        mats[mat] = (w, _gpu_weights(w, quant.W4_SYM, 64))
    yield c, mats
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", [64, 256, 1024])
def test_prefill_w4_4096(prefill_w4_4096, m):
    c, mats = prefill_w4_4096
    for mat, n, k in synth.layer_shapes(c):
        x = synth.act_normal(m, k, 3, salt=20 + mat)
        y = torch.empty(m * n * 2, dtype=torch.uint8, device="cuda")
        say("prefill w4 4096", synth.MAT_NAMES[mat], "m", m)
        rq.rq_gemm_w4(dev_f16(x), m, k, mats[mat][1], y, n)
        torch.cuda.synchronize()
        rows = _rows(n, 700 + mat + m)
        parts = _check_rows_sym(mats[mat][1], mats[mat][0], rows, quant.W4_SYM, 64)
        _compare_rows(host(y, np.float16).reshape(m, n), rows, x, quant.W4_SYM, parts, 64,
                      synth.MAT_NAMES[mat])


@pytest.mark.parametrize("m", [64, 256, 1024])
def test_prefill_sb256_4096(m):
    """The width-4096 prefill set on asymmetric superblock codes (rq_gemm_w4)."""
    c = 4096
    for mat, n, k in synth.layer_shapes(c):
        w = synth.weight(3, 20, mat, n, k)
        qw = _gpu_weights(w, quant.W4_ASYM_SB256, 32)
        x = synth.act_normal(m, k, 3, salt=40 + mat)
        y = torch.empty(m * n * 2, dtype=torch.uint8, device="cuda")
        say("prefill sb256 4096", synth.MAT_NAMES[mat], "m", m)
        rq.rq_gemm_w4(dev_f16(x), m, k, qw, y, n)
        torch.cuda.synchronize()
        rows = _rows(n, 800 + mat + m)
        parts = _check_rows_sb(qw, w, rows)
        _compare_rows(host(y, np.float16).reshape(m, n), rows, x, quant.W4_ASYM_SB256, parts, 32,
                      synth.MAT_NAMES[mat])
        del qw


# --------------------------------------------------------------------------
# width 4096 (13.3B) decode step: one layer's six matrices (every layer has
# these shapes) at M in {1, 2, 4, 8, 16, 32}, and the fp16 head
# --------------------------------------------------------------------------


@pytest.fixture(scope="module")
def layer_4096():
    c = 4096
    mats = {}
    for mat, n, k in synth.layer_shapes(c):
        w = synth.weight(4, 60, mat, n, k)
        mats[mat] = (w, _gpu_weights(w, quant.W4_SYM, 64))
    yield c, mats
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", [1, 2, 3, 4, 6, 8, 9, 12, 16, 17, 24, 32])
def test_decode_layer_4096(layer_4096, m):
    c, mats = layer_4096
    x = synth.act_normal(m, c, 4)
    x4 = synth.act_normal(m, 4 * c, 4, salt=1)
    xd, x4d = dev_f16(x), dev_f16(x4)
    q = {mat: mats[mat][1] for mat in mats}
    ys = {mat: torch.empty(m * n * 2, dtype=torch.uint8, device="cuda") for mat, n, _ in synth.layer_shapes(c)}
    say("decode layer 4096 m", m)
    rq.rq_fused_rkv(xd, xd, xd, m, c, q[synth.MAT_R], q[synth.MAT_K], q[synth.MAT_V],
                    ys[synth.MAT_R], ys[synth.MAT_K], ys[synth.MAT_V], c)
    rq.rq_gemm_small_m(xd, m, c, q[synth.MAT_O], ys[synth.MAT_O], c)
    rq.rq_gemm_small_m(xd, m, c, q[synth.MAT_KEY], ys[synth.MAT_KEY], 4 * c)
    rq.rq_gemm_small_m(x4d, m, 4 * c, q[synth.MAT_VALUE], ys[synth.MAT_VALUE], c)
    torch.cuda.synchronize()
    for mat, n, k in synth.layer_shapes(c):
        rows = _rows(n, 500 + mat + m)
        parts = _check_rows_sym(q[mat], mats[mat][0], rows, quant.W4_SYM, 64)
        _compare_rows(host(ys[mat], np.float16).reshape(m, n), rows, x4 if k == 4 * c else x,
                      quant.W4_SYM, parts, 64, synth.MAT_NAMES[mat])


@pytest.fixture(scope="module")
def head_4096():
    n, k = 65536, 4096
    w = synth.weight(4, 61, synth.MAT_HEAD, n, k)
    qw = _gpu_weights(w, quant.F16, 0)
    rows = _rows(n, 600)
    parts = {"codes": w[rows].astype(np.float16)}
    assert np.array_equal(host(qw.codes, np.uint16)[: n * k].reshape(n, k)[rows], parts["codes"].view(np.uint16))
    yield qw, rows, parts
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_head_4096x65536(head_4096, m):
    n, k = 65536, 4096
    qw, rows, parts = head_4096
    x = synth.act_normal(m, k, 4, salt=2)
    y = torch.empty(m * n * 2, dtype=torch.uint8, device="cuda")
    say("head m", m)
    if m == 1:
        rq.rq_gemv_f16(dev_f16(x), qw, y)
    else:
        rq.rq_gemm_small_m(dev_f16(x), m, k, qw, y, n)
    torch.cuda.synchronize()
    _compare_rows(host(y, np.float16).reshape(m, n), rows, x, quant.F16, parts, 0, "head")


# --------------------------------------------------------------------------
# a reduced 13.3B decode step in one graph: two width-4096 layers and the
# head, launched as the benchmark's sweep launches them (fused R/K/V, O, cmix
# key, cmix value per layer, then the head), captured once per M, replayed,
# and checked on sampled rows of every output
# --------------------------------------------------------------------------


@pytest.fixture(scope="module")
def step_4096(layer_4096, head_4096):
    c, mats = layer_4096
    second = {}
    for mat, n, k in synth.layer_shapes(c):
        w = synth.weight(4, 59, mat, n, k)
        second[mat] = (w, _gpu_weights(w, quant.W4_SYM, 64))
    yield c, [mats, second], head_4096
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_step_graph_4096(step_4096, m):
    c, layers, (qh, hrows, hparts) = step_4096
    x = synth.act_normal(m, c, 4, salt=3)
    x4 = synth.act_normal(m, 4 * c, 4, salt=4)
    xd, x4d = dev_f16(x), dev_f16(x4)
    shapes = synth.layer_shapes(c)
    ys = [{mat: torch.zeros(m * n, dtype=torch.int16, device="cuda") for mat, n, _ in shapes} for _ in layers]
    yh = torch.zeros(m * 65536, dtype=torch.int16, device="cuda")

    def step():
        for li, mats in enumerate(layers):
            q = {mat: mats[mat][1] for mat in mats}
            y = ys[li]
            rq.rq_fused_rkv(xd, xd, xd, m, c, q[synth.MAT_R], q[synth.MAT_K], q[synth.MAT_V],
                            y[synth.MAT_R], y[synth.MAT_K], y[synth.MAT_V], c)
            rq.rq_gemm_small_m(xd, m, c, q[synth.MAT_O], y[synth.MAT_O], c)
            rq.rq_gemm_small_m(xd, m, c, q[synth.MAT_KEY], y[synth.MAT_KEY], 4 * c)
            rq.rq_gemm_small_m(x4d, m, 4 * c, q[synth.MAT_VALUE], y[synth.MAT_VALUE], c)
        rq.rq_gemm_small_m(xd, m, c, qh, yh, 65536)

    rq.default_workspace()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("step graph 4096 capture m", m)
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for y in ys:
            for t in y.values():
                t.fill_(-1)
        yh.fill_(-1)
        torch.cuda.synchronize()
        say("step graph 4096 replay m", m, rep)
        g.replay()
        torch.cuda.synchronize()
        for li, mats in enumerate(layers):
            for mat, n, k in shapes:
                rows = _rows(n, 900 + 10 * li + mat + m)
                parts = _check_rows_sym(mats[mat][1], mats[mat][0], rows, quant.W4_SYM, 64)
                _compare_rows(host(ys[li][mat], np.float16).reshape(m, n), rows, x4 if k == 4 * c else x,
                              quant.W4_SYM, parts, 64, (li, synth.MAT_NAMES[mat], rep))
        _compare_rows(host(yh, np.float16).reshape(m, 65536), hrows, x, quant.F16, hparts, 0, ("head", rep))
    del g


@pytest.mark.parametrize("fmt,group,n,k,mat", [(quant.W4_SYM, 64, 4096, 4096, synth.MAT_O),
                                               (quant.W4_ASYM_SB256, 32, 2560, 10240, synth.MAT_VALUE),
                                               (quant.W8_SYM, 32, 10240, 2560, synth.MAT_KEY)])
def test_quantize_aw_fullsize(fmt, group, n, k, mat):
    """rq_quantize_aw on whole matrices of the 2.9B and 4096-wide layers with
    E[x^2] from a massive-channel calibration batch; the sampled rows' bytes
    equal the oracle's AW search of those rows (each row depends on itself
    and the shared importance only)."""
    from oracle import aw
    w = synth.weight(2, 3, mat, n, k)
    xc = synth.act_massive(256, k, cfg=2, salt=11).astype(np.float64)
    a = np.mean(xc * xc, axis=0).astype(np.float32)
    say("quantize_aw full", fmt, group, n, k)
    qw = rq.quantize_aw(dev_f32(w), dev_f32(a), fmt, group)
    torch.cuda.synchronize()
    rows = _rows(n, 77)
    parts = aw.quantize_aw(w[rows], a, fmt, group)
    assert np.any(parts["t"] > 0)
    got = qw.buffers()
    if fmt == quant.W4_ASYM_SB256:
        nsb = k // 256
        pairs = (("codes", parts["qs"], k // 2), ("scales", parts["d"], nsb * 2),
                 ("mins", parts["dmin"], nsb * 2), ("sub", parts["sub"], nsb * 12))
    else:
        cb = k // 2 if fmt == quant.W4_SYM else k
        pairs = (("codes", parts["codes"], cb), ("scales", parts["scales"], (k // group) * 2))
    for name, want, row_bytes in pairs:
        g = host(got[name], np.uint8).reshape(n, row_bytes)[rows]
        assert np.array_equal(g, np.ascontiguousarray(want).reshape(len(rows), -1).view(np.uint8)), name
