"""GPU parity of the preset widths: 6- and 5-bit symmetric group codes (two
planes) and bfloat16 weights, against the oracle.

Quantizers (RTN and activation-weighted) must give the oracle's bytes; the
weight-streaming products (rq_gemm_small_m, rq_fused_rkv) must meet the
tolerance of oracle.ref.compare and be exact on integer cases.  Expected
values come only from oracle/.
"""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import synth
from gpu_helpers import dev_f16, dev_f32, host, oracle_buffers, qweight_from_oracle, random_parts, say
from oracle import aw, quant, ref

pytestmark = pytest.mark.gpu

W56 = [(quant.W6_SYM, 32), (quant.W6_SYM, 64), (quant.W5_SYM, 32), (quant.W5_SYM, 64)]


def _weights(n, k, seed, kind="normal"):
    g = np.random.default_rng(seed)
    if kind == "normal":
        return (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    w = (g.standard_normal((n, k)) * 10.0 ** g.uniform(-7, 3, (n, 1))).astype(np.float32)
    if n > 4 and k >= 64:
        w[0, :64] = 0
        w[1, :32] = 0.37
        w[2, :32] = -1.25
        w[3, 7] = 3e3
        w[4, 32:64] = -0.0
    return w


def _compare_bytes(qw, fmt, parts, what):
    got = qw.buffers()
    for name, arr in oracle_buffers(fmt, parts).items():
        g = host(got[name], np.uint8)
        wb = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
        if not np.array_equal(g, wb):
            bad = np.nonzero(g != wb)[0]
            raise AssertionError("%s %s: %d bytes differ, first at %d (got %d want %d)"
                                 % (what, name, len(bad), bad[0], g[bad[0]], wb[bad[0]]))


@pytest.mark.parametrize("fmt,group", W56)
@pytest.mark.parametrize("n,k,kind", [(7, 256, "normal"), (65, 512, "adversarial"),
                                      (200, 1024, "normal"), (33, 2560, "adversarial")])
def test_quantize_56_bytes_exact(fmt, group, n, k, kind):
    w = _weights(n, k, seed=n * 11 + k, kind=kind)
    parts = quant.quantize(w, fmt, group)
    say("quantize", fmt, group, n, k)
    qw = rq.quantize(dev_f32(w), fmt, group)
    torch.cuda.synchronize()
    _compare_bytes(qw, fmt, parts, "rtn fmt %d g %d" % (fmt, group))
    # the activation-weighted search on the same weights
    g = np.random.default_rng(k)
    a = g.exponential(1.0, k)
    a[g.choice(k, 3, replace=False)] = 2500.0
    a = a.astype(np.float32)
    parts = aw.quantize_aw(w, a, fmt, group)
    say("quantize_aw", fmt, group, n, k)
    qw = rq.quantize_aw(dev_f32(w), dev_f32(a), fmt, group)
    torch.cuda.synchronize()
    _compare_bytes(qw, fmt, parts, "aw fmt %d g %d" % (fmt, group))


def test_quantize_bf16_bytes_exact():
    g = np.random.default_rng(3)
    w = (g.standard_normal((64, 256)) * 10.0 ** g.uniform(-40, 37, (64, 1))).astype(np.float32)
    top = g.integers(0, 0x7F7F, (8, 256)).astype(np.uint32) << 16
    w[:8] = (top | 0x8000).view(np.float32)            # exact ties between two bf16 values
    w[8:16] = -w[:8]
    w[16, :4] = [0.0, -0.0, 1e-45, 3.3895314e38]
    parts = quant.quantize(w, quant.BF16)
    say("quantize bf16", w.shape)
    qw = rq.quantize(dev_f32(w), quant.BF16)
    torch.cuda.synchronize()
    _compare_bytes(qw, quant.BF16, parts, "bf16")


def test_quantize_56_bf16_errors():
    w = _weights(4, 128, 1)
    w[1, 2] = np.nan
    for fmt, group in ((quant.W6_SYM, 32), (quant.BF16, 0)):
        with pytest.raises(rq.RqError) as e:
            rq.quantize(dev_f32(w), fmt, group)
        assert e.value.status == rq.RQ_ERR_NONFINITE
    big = np.full((2, 128), 3.4e38, np.float32)
    with pytest.raises(rq.RqError) as e:
        rq.quantize(dev_f32(big), quant.BF16)
    assert e.value.status == rq.RQ_ERR_RANGE


def _run_small_m(qw, x, m, ldx, n):
    y = torch.zeros(m * n, dtype=torch.int16, device="cuda")
    xd = dev_f16(x)
    say("small_m", qw.format, qw.group, n, qw.k, m)
    rq.rq_gemm_small_m(xd, m, ldx, qw, y, n)
    torch.cuda.synchronize()
    return host(y, np.float16, (m, n)).astype(np.float64)


@pytest.mark.parametrize("fmt,group", W56 + [(quant.BF16, 0)])
@pytest.mark.parametrize("n,k", [(3, 128), (1, 256), (7, 512), (65, 768), (160, 2048), (48, 8192)])
@pytest.mark.parametrize("m", [1, 2, 5, 16, 17, 32])
def test_small_m_56_bf16_parity(fmt, group, n, k, m):
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


@pytest.mark.parametrize("fmt,group", W56)
def test_56_integer_special_case_exact(fmt, group):
    """Integer codes with one +-Q per group have scale 1, so W_hat holds small
    integers; with integer activations every product and partial sum is an
    integer below 2^24 and the fp16 output is the exact sum rounded once."""
    n, k, m = 96, 1024, 8
    bits = quant.SYM_BITS[fmt]
    Q = (1 << (bits - 1)) - 1
    g = np.random.default_rng(bits * 10 + group)
    q = g.integers(-Q, Q + 1, (n, k))
    q.reshape(n, k // group, group)[..., 0] = Q
    parts = quant.quantize(q.astype(np.float32), fmt, group)
    assert np.all(parts["scales"] == 1.0)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    x = g.integers(-3, 4, (m, k)).astype(np.float16)
    y = _run_small_m(qw, x, m, k, n)
    want = (x.astype(np.float64) @ q.astype(np.float64).T).astype(np.float16).astype(np.float64)
    assert np.array_equal(y, want)


def test_bf16_integer_special_case_exact():
    # weights are small integers (exact in bf16); activations j / 256 with up
    # to 11 significant bits, so the kernel's hi + lo split of x is exercised;
    # every partial sum is a multiple of 2^-8 below 2^15, exact in fp32
    n, k, m = 64, 256, 4
    g = np.random.default_rng(8)
    w = g.integers(-16, 17, (n, k)).astype(np.float32)
    parts = quant.quantize(w, quant.BF16)
    qw = qweight_from_oracle(quant.BF16, 0, parts, n, k)
    x = (g.integers(-2047, 2048, (m, k)) / 256.0).astype(np.float16)
    y = _run_small_m(qw, x, m, k, n)
    want = (x.astype(np.float64) @ w.astype(np.float64).T).astype(np.float16).astype(np.float64)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("fmt,group", [(quant.W6_SYM, 64), (quant.W5_SYM, 32)])
def test_fused_rkv_56(fmt, group):
    c, m = 768, 4
    ws = [_weights(c, c, seed=40 + i) for i in range(3)]
    parts = [quant.quantize(w, fmt, group) for w in ws]
    qws = [qweight_from_oracle(fmt, group, p, c, c) for p in parts]
    g = np.random.default_rng(5)
    xs = [g.standard_normal((m, c)).astype(np.float16) for _ in range(3)]
    xd = [dev_f16(x) for x in xs]
    ys = [torch.zeros(m * c, dtype=torch.int16, device="cuda") for _ in range(3)]
    say("fused_rkv", fmt, group, c, m)
    rq.rq_fused_rkv(xd[0], xd[1], xd[2], m, c, qws[0], qws[1], qws[2], ys[0], ys[1], ys[2], c)
    torch.cuda.synchronize()
    for x, p, y in zip(xs, parts, ys):
        y_ref, b = ref.weight_only_ref(x, fmt, p, group)
        ok, info = ref.compare(host(y, np.float16, (m, c)).astype(np.float64), y_ref, b)
        assert ok, info


def test_56_product_on_gpu_quantized_weights_fullsize():
    """The 2.9B-width channel-mix matrices quantized on the GPU (6-bit g32
    value, 5-bit g32 key) and the layer-0 output projection in bf16, each
    multiplied at M = 1, 4, 16; sampled rows against the oracle."""
    for fmt, group, n, k, mat in ((quant.W6_SYM, 32, 2560, 10240, synth.MAT_VALUE),
                                  (quant.W5_SYM, 32, 10240, 2560, synth.MAT_KEY),
                                  (quant.BF16, 0, 2560, 2560, synth.MAT_O)):
        w = synth.weight(2, 0, mat, n, k)
        say("fullsize quantize", fmt, group, n, k)
        qw = rq.quantize(dev_f32(w), fmt, group)
        rows = np.sort(np.random.default_rng(n).choice(n, 40, replace=False))
        parts = quant.quantize(w[rows], fmt, group)
        got = qw.buffers()
        for name, arr in oracle_buffers(fmt, parts).items():
            per_row = got[name].numel() // n
            g = host(got[name], np.uint8).reshape(n, per_row)[rows]
            assert np.array_equal(g, np.ascontiguousarray(arr).reshape(len(rows), -1).view(np.uint8)), name
        for m in (1, 4, 16):
            x = synth.act_massive(m, k, cfg=2, salt=m)
            y = _run_small_m(qw, x, m, k, n)[:, rows]
            y_ref, b = ref.weight_only_ref(x, fmt, parts, group)
            ok, info = ref.compare(y, y_ref, b)
            assert ok, (fmt, m, info)


def test_56_bf16_shape_limit():
    """The 6-/5-bit and bf16 products have one kernel: K may be cut into at
    most 16 slices, whose activation slices must fit LDS.  At m = 32,
    k = 18432 is the largest 6-bit K that fits; k = 25600 is refused with
    RQ_ERR_SHAPE and leaves the output untouched."""
    n, m = 64, 32
    for k, fits in ((18432, True), (25600, False)):
        g = np.random.default_rng(k)
        parts = random_parts(quant.W6_SYM, 32, n, k, g)
        qw = qweight_from_oracle(quant.W6_SYM, 32, parts, n, k)
        x = g.standard_normal((m, k)).astype(np.float16)
        say("w6 limit", k, fits)
        if fits:
            y = _run_small_m(qw, x, m, k, n)
            y_ref, b = ref.weight_only_ref(x, quant.W6_SYM, parts, 32)
            ok, info = ref.compare(y, y_ref, b)
            assert ok, info
        else:
            y = torch.full((m * n,), 7, dtype=torch.int16, device="cuda")
            with pytest.raises(rq.RqError) as e:
                rq.rq_gemm_small_m(dev_f16(x), m, k, qw, y, n)
            assert e.value.status == rq.RQ_ERR_SHAPE
            torch.cuda.synchronize()
            assert bool((y == 7).all())
