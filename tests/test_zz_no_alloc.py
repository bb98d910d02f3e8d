"""rq_gemm_small_m_noalloc (static device scratch, allocates nothing) against
rq_gemm_small_m with a full workspace and against the oracle.

Two calls in a row on the same GPU share the scratch: the second, smaller
product must not see the first one's partial sums.  Shapes cut K across
workgroups (their partial sums go through the scratch) and one does not."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import synth
from gpu_helpers import dev_f16, host, qweight_from_oracle, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu


def _case(fmt, group, n, k, m, seed):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    parts = quant.quantize(w, fmt, group)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    x = synth.act_channel_1202(m, k) if k > 1202 else g.standard_normal((m, k)).astype(np.float16)
    return parts, qw, x


@pytest.mark.parametrize("first,second", [
    # (format, group, n, k, m): the first call leaves partial sums of a K split in the scratch
    ((quant.W4_SYM, 64, 2048, 8192, 32), (quant.W4_SYM, 64, 1024, 4096, 8)),
    ((quant.W4_ASYM_SB256, 32, 2560, 10240, 16), (quant.W4_ASYM_SB256, 32, 640, 2560, 4)),
    ((quant.W8_SYM, 64, 4096, 16384, 4), (quant.W8_SYM, 64, 512, 2048, 1)),
    ((quant.W6_SYM, 32, 2048, 8192, 17), (quant.W5_SYM, 32, 256, 1024, 3)),
])
def test_noalloc_matches_workspace_entry(first, second):
    for call, (fmt, group, n, k, m) in enumerate((first, second)):
        parts, qw, x = _case(fmt, group, n, k, m, seed=31 + call + n)
        xd = dev_f16(x)
        y0 = torch.full((m * n,), -1, dtype=torch.int16, device="cuda")
        y1 = torch.full((m * n,), -1, dtype=torch.int16, device="cuda")
        say("noalloc call", call, fmt, group, n, k, m)
        rq.rq_gemm_small_m(xd, m, k, qw, y0, n)                 # the binding's full workspace
        rq.rq_gemm_small_m_noalloc(xd, m, k, qw, y1, n)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), ("noalloc differs from the workspace entry", call, fmt, n, k, m)
        y_ref, b = ref.weight_only_ref(x, fmt, parts, group)
        ok, info = ref.compare(host(y1, np.float16, (m, n)).astype(np.float64), y_ref, b)
        assert ok, (call, fmt, n, k, m, info)


def test_noalloc_refuses_beyond_scratch():
    parts, qw, x = _case(quant.W4_SYM, 64, 4112, 1024, 17, seed=5)
    y = torch.zeros(17 * 4112, dtype=torch.int16, device="cuda")
    with pytest.raises(rq.RqError) as e:
        rq.rq_gemm_small_m_noalloc(dev_f16(x), 17, 1024, qw, y, 4112)
    assert e.value.status == rq.RQ_ERR_SCRATCH
