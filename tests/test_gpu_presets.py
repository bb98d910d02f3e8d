"""One 2.9B-shape layer (width 2560) and the head under each rwkv-quant preset
(gemm_rwkv_amd.presets): weights quantized on the GPU in the preset's format
per tensor, then the decode launches bench.py's preset sweep times (fused
R/K/V, O, cmix key, cmix value, head) at the sweep's M = 1, 4 and 16.  Sampled rows of every
quantized tensor are checked byte for byte against the oracle, and their
outputs against the oracle's product."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import presets, synth
from gpu_helpers import dev_f16, dev_f32, host, oracle_buffers, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu

C, VOCAB = 2560, 65536
SHAPES = {"r": (C, C), "k": (C, C), "v": (C, C), "o": (C, C), "cmix_key": (4 * C, C),
          "cmix_value": (C, 4 * C), "head": (VOCAB, C)}
MAT = {"r": synth.MAT_R, "k": synth.MAT_K, "v": synth.MAT_V, "o": synth.MAT_O, "cmix_key": synth.MAT_KEY,
       "cmix_value": synth.MAT_VALUE, "head": synth.MAT_HEAD}


def _check(qw, w, fmt, group, rows, x, y):
    parts = quant.quantize(w[rows], fmt, group)
    got = qw.buffers()
    n = w.shape[0]
    for name, arr in oracle_buffers(fmt, parts).items():
        per_row = got[name].numel() // n
        g = host(got[name], np.uint8).reshape(n, per_row)[rows]
        assert np.array_equal(g, np.ascontiguousarray(arr).reshape(len(rows), -1).view(np.uint8)), name
    y_ref, b = ref.weight_only_ref(x, fmt, parts, group)
    ok, info = ref.compare(host(y, np.float16, (x.shape[0], n))[:, rows].astype(np.float64), y_ref, b)
    assert ok, info


@pytest.fixture(scope="module")
def weights_2560():
    return {t: synth.weight(2, 0, MAT[t], *SHAPES[t]) for t in presets.TENSORS}


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("preset,bf16_o0", [("REDUCTION", False), ("COMPRESSION", False),
                                            ("COMPRESSION", True)])
def test_preset_layer_and_head(weights_2560, preset, bf16_o0, M):
    x = synth.act_massive(M, C, cfg=2, salt=1)
    x4 = synth.act_massive(M, 4 * C, cfg=2, salt=2)
    xd, x4d = dev_f16(x), dev_f16(x4)
    ws, qws, ys = weights_2560, {}, {}
    for t in presets.TENSORS:
        n, k = SHAPES[t]
        fmt, group = presets.scheme(preset, t, 0, bf16_o0)
        say("preset", preset, bf16_o0, t, fmt, group, n, k)
        qws[t] = rq.quantize(dev_f32(ws[t]), fmt, group)
        ys[t] = torch.zeros(M * n, dtype=torch.int16, device="cuda")
    rq.rq_fused_rkv(xd, xd, xd, M, C, qws["r"], qws["k"], qws["v"], ys["r"], ys["k"], ys["v"], C)
    rq.rq_gemm_small_m(xd, M, C, qws["o"], ys["o"], C)
    rq.rq_gemm_small_m(xd, M, C, qws["cmix_key"], ys["cmix_key"], 4 * C)
    rq.rq_gemm_small_m(x4d, M, 4 * C, qws["cmix_value"], ys["cmix_value"], C)
    rq.rq_gemm_small_m(xd, M, C, qws["head"], ys["head"], VOCAB)
    torch.cuda.synchronize()
    for t in presets.TENSORS:
        n, k = SHAPES[t]
        fmt, group = presets.scheme(preset, t, 0, bf16_o0)
        rows = np.sort(np.random.default_rng(n + k).choice(n, 24, replace=False))
        _check(qws[t], ws[t], fmt, group, rows, x4 if t == "cmix_value" else x, ys[t])
