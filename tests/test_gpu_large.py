"""Weights past 2 GiB in one buffer.  The streaming kernel addresses its
buffers with 32-bit buffer resources, so such a matrix takes the first
kernel (64-bit addressing) for the int4/int8/SB256/fp16 formats and is
refused with RQ_ERR_SHAPE for the formats that have no other kernel.  Codes
and scales are random bytes drawn on the GPU (inputs, not results); sampled
rows are copied back and multiplied by the oracle."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_f16, host, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu


def test_int4_codes_past_2gib():
    n, k, m = 40000, 131072, 2                      # 2.62 GB of int4 codes
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    say("large int4", n, k, m)
    codes = torch.randint(0, 256, (n * k // 2,), dtype=torch.uint8, device="cuda", generator=g)
    # fp16 scales in [2^-10, 2^-9): exponent field 5, random mantissa
    sbits = (torch.randint(0, 1024, (n * (k // 64),), dtype=torch.int32, device="cuda", generator=g) | (5 << 10))
    scales = sbits.to(torch.int16).view(torch.uint8)
    qw = rq.QWeight(rq.RQ_W4_SYM, 64, n, k, codes, scales)
    x = np.random.default_rng(1).standard_normal((m, k)).astype(np.float16)
    y = torch.zeros(m * n, dtype=torch.int16, device="cuda")
    rq.rq_gemm_small_m(dev_f16(x), m, k, qw, y, n)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(2).choice(n, 16, replace=False))
    rows = np.concatenate([rows, [n - 1]])
    cb = codes.view(n, k // 2)[torch.from_numpy(rows).cuda()].cpu().numpy()
    sb = scales.view(n, (k // 64) * 2)[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.float16)
    parts = {"codes": cb, "scales": sb}
    y_ref, b = ref.weight_only_ref(x, quant.W4_SYM, parts, 64)
    got = host(y, np.float16, (m, n))[:, rows].astype(np.float64)
    ok, info = ref.compare(got, y_ref, b)
    assert ok, info


def test_bf16_past_2gib_is_refused():
    n, k = 32768, 32768                            # 2 GiB of bf16
    w = rq.QWeight(rq.RQ_BF16, 0, n, k, torch.empty(n * k * 2, dtype=torch.uint8, device="cuda"))
    x = torch.zeros(k * 2, dtype=torch.uint8, device="cuda")
    y = torch.zeros(n, dtype=torch.int16, device="cuda")
    say("large bf16 refused", n, k)
    with pytest.raises(rq.RqError) as e:
        rq.rq_gemm_small_m(x, 1, k, w, y, n)
    assert e.value.status == rq.RQ_ERR_SHAPE
