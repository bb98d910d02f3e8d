"""GPU parity of the activation-weighted (AW) quantizer (rq_quantize_aw)
against oracle/aw.py: codes, scales, mins and sub-codes byte-equal.

Importances are E[x^2]-like vectors: a seeded exponential spread with a few
channels 2500 times larger, or the mean square of a batch of massive-channel
activations from gemm_rwkv_amd.synth.  Expected values come only from oracle/.
"""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import synth
from gpu_helpers import dev_f32, host, oracle_buffers, say
from oracle import aw, quant

pytestmark = pytest.mark.gpu

FORMATS = [(quant.W4_SYM, 64), (quant.W4_SYM, 32), (quant.W4_SYM, 16),
           (quant.W8_SYM, 64), (quant.W8_SYM, 32), (quant.W8_SYM, 16),
           (quant.W4_ASYM_SB256, 32)]


def _weights(n, k, seed, kind="normal"):
    g = np.random.default_rng(seed)
    if kind == "normal":
        w = g.standard_normal((n, k)) / np.sqrt(k)
        w[0, :8] *= 6.0
        return w.astype(np.float32)
    # adversarial: row magnitudes over many decades, zero / constant / signed-zero groups
    w = (g.standard_normal((n, k)) * 10.0 ** g.uniform(-7, 3, (n, 1))).astype(np.float32)
    if n > 4 and k >= 64:
        w[0, :64] = 0
        w[1, :32] = 0.37
        w[2, :32] = -1.25
        w[3, 7] = 3e3
        w[4, 32:64] = -0.0
    return w


def _importance(k, seed, zero_block=False):
    g = np.random.default_rng(seed)
    a = g.exponential(1.0, k)
    a[g.choice(k, min(3, k), replace=False)] = 2500.0
    if zero_block:
        a[:64] = 0.0          # whole groups without weight: every candidate scores 0
        a[100:103] = 0.0
    return a.astype(np.float32)


def _aw_gpu(w, a, fmt, group):
    n, k = w.shape
    say("quantize_aw", fmt, group, n, k)
    qw = rq.quantize_aw(dev_f32(w), dev_f32(a), fmt, group)
    torch.cuda.synchronize()
    return qw


def _compare(qw, fmt, parts, what=""):
    got = qw.buffers()
    for name, arr in oracle_buffers(fmt, parts).items():
        g = host(got[name], np.uint8)
        wb = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
        if not np.array_equal(g, wb):
            bad = np.nonzero(g != wb)[0]
            raise AssertionError("%s %s: %d bytes differ, first at %d (got %d want %d)"
                                 % (what, name, len(bad), bad[0], g[bad[0]], wb[bad[0]]))


@pytest.mark.parametrize("fmt,group", FORMATS)
@pytest.mark.parametrize("n,k,kind", [(7, 256, "normal"), (65, 512, "adversarial"),
                                      (200, 1024, "normal"), (33, 2560, "adversarial")])
def test_aw_bytes_exact(fmt, group, n, k, kind):
    w = _weights(n, k, seed=n * 3 + k, kind=kind)
    a = _importance(k, seed=k + n, zero_block=(kind == "adversarial"))
    parts = aw.quantize_aw(w, a, fmt, group)
    assert np.any(parts["t"] > 0)                  # the search moved some group
    _compare(_aw_gpu(w, a, fmt, group), fmt, parts, "fmt %d g %d" % (fmt, group))


@pytest.mark.parametrize("fmt,group", [(quant.W4_SYM, 64), (quant.W8_SYM, 16), (quant.W4_ASYM_SB256, 32)])
def test_aw_zero_importance_is_rtn(fmt, group):
    w = _weights(48, 768, seed=5)
    a = np.zeros(768, np.float32)
    parts = quant.quantize(w, fmt, group)
    _compare(_aw_gpu(w, a, fmt, group), fmt, parts, "zero importance")
    # and the same bytes as the library's own RTN
    rtn = rq.quantize(dev_f32(w), fmt, group).buffers()
    got = _aw_gpu(w, a, fmt, group).buffers()
    for name in rtn:
        if rtn[name] is not None:
            assert torch.equal(rtn[name], got[name]), name


@pytest.mark.parametrize("fmt,group", [(quant.W4_SYM, 64), (quant.W4_ASYM_SB256, 32)])
def test_aw_massive_channel_importance(fmt, group):
    """Importance from a calibration batch of massive-channel activations at
    the 2.9B model width (K = 2560, 10240 for the channel-mix value)."""
    for n, k, mat in ((512, 2560, synth.MAT_O), (256, 10240, synth.MAT_VALUE)):
        w = synth.weight(2, 1, mat, n, k)
        xc = synth.act_massive(128, k, cfg=2, salt=7).astype(np.float64)
        a = np.mean(xc * xc, axis=0).astype(np.float32)
        parts = aw.quantize_aw(w, a, fmt, group)
        _compare(_aw_gpu(w, a, fmt, group), fmt, parts, "massive %dx%d" % (n, k))


def test_aw_signed_zero_and_constant_groups():
    g = np.random.default_rng(4)
    w = np.zeros((4, 512), np.float32)
    w[0] = np.abs(g.standard_normal(512)).astype(np.float32) + 0.25
    w[1] = -0.0
    w[2, :256] = -0.0
    w[2, 256:] = g.standard_normal(256).astype(np.float32)
    w[3, :32] = 0.5
    w[3, 32:] = -np.abs(g.standard_normal(480)).astype(np.float32)
    a = _importance(512, 9)
    for fmt, group in ((quant.W4_ASYM_SB256, 32), (quant.W4_SYM, 32), (quant.W8_SYM, 64)):
        parts = aw.quantize_aw(w, a, fmt, group)
        _compare(_aw_gpu(w, a, fmt, group), fmt, parts, "fmt %d" % fmt)


def test_aw_errors():
    w = _weights(8, 256, seed=1)
    a = _importance(256, 2)
    bad = a.copy()
    bad[17] = np.nan
    with pytest.raises(rq.RqError) as e:
        _aw_gpu(w, bad, quant.W4_SYM, 64)
    assert e.value.status == rq.RQ_ERR_NONFINITE
    bad = a.copy()
    bad[200] = -1.0
    with pytest.raises(rq.RqError) as e:
        _aw_gpu(w, bad, quant.W4_ASYM_SB256, 32)
    assert e.value.status == rq.RQ_ERR_NONFINITE
    wn = w.copy()
    wn[2, 3] = np.inf
    with pytest.raises(rq.RqError) as e:
        _aw_gpu(wn, a, quant.W8_SYM, 32)
    assert e.value.status == rq.RQ_ERR_NONFINITE
    with pytest.raises(rq.RqError) as e:
        _aw_gpu(np.full((2, 64), 3e38, np.float32), a[:64], quant.W4_SYM, 64)
    assert e.value.status == rq.RQ_ERR_RANGE
    # a NaN importance must not reach the output of a clean call that follows
    parts = aw.quantize_aw(w, a, quant.W4_SYM, 64)
    _compare(_aw_gpu(w, a, quant.W4_SYM, 64), quant.W4_SYM, parts, "after errors")


def test_aw_product_parity():
    """AW codes go through the unchanged product kernels: the GEMV on them
    matches the oracle's product of the oracle's AW codes, and on
    massive-channel inputs its error against the unquantized product is
    below that of the same kernel on RTN codes."""
    from gpu_helpers import dev_f16
    from oracle import ref
    n, k, m = 256, 2560, 8
    w = synth.weight(2, 2, synth.MAT_O, n, k)
    xc = synth.act_massive(64, k, cfg=2, salt=3).astype(np.float64)
    a = np.mean(xc * xc, axis=0).astype(np.float32)
    x = synth.act_massive(m, k, cfg=2, salt=4)
    for fmt, group, name in ((quant.W4_SYM, 64, "rq_gemv_w4g64"), (quant.W4_ASYM_SB256, 32, "rq_gemv_w4sb256")):
        parts = aw.quantize_aw(w, a, fmt, group)
        qw = _aw_gpu(w, a, fmt, group)
        xd = dev_f16(x)
        y = torch.empty(m * n * 2, dtype=torch.uint8, device="cuda")
        say(name, n, k, m)
        rq.rq_gemm_small_m(xd, m, k, qw, y, n)
        torch.cuda.synchronize()
        yr, bound = ref.weight_only_ref(x, fmt, parts, group)
        y_aw = host(y, np.float16, (m, n)).astype(np.float64)
        ok, info = ref.compare(y_aw, yr, bound)
        assert ok, (name, info)
        qr = rq.quantize(dev_f32(w), fmt, group)
        rq.rq_gemm_small_m(xd, m, k, qr, y, n)
        torch.cuda.synchronize()
        y_rtn = host(y, np.float16, (m, n)).astype(np.float64)
        y_fp = x.astype(np.float64) @ w.astype(np.float64).T
        assert np.linalg.norm(y_aw - y_fp) < 0.9 * np.linalg.norm(y_rtn - y_fp), name
