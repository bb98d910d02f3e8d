"""int4 products at M = 1 on matrices of fewer than 256 row tiles of 16,
where each 8-row tile covers K as two ranges (the MFMA's diagonal blocks):
tile counts from one to 255, ragged last tiles (n not a multiple of 8 or 16),
ranges of 16 to 64 chunks with ragged waves, both int4 groups, fused R/K/V
with three small matrices, and K of fewer than 32 chunks or a chunk count
that is not a multiple of eight (the one-range plan).  Every output row is compared with the oracle,
and the bytes after n must stay untouched."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_f16, host, qweight_from_oracle, random_parts, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu

# two ranges from 32 chunks (K = 4096) when the chunk count is a multiple of
# eight; (2048, 2048) and (300, 1536) take the one-range plan
SHAPES = [(2048, 8192), (1000, 4096), (8, 4096), (9, 5120), (136, 5120), (4072, 4096), (2040, 16384),
          (2048, 2048), (300, 1536)]


def _run(fmt, group, n, k, seed):
    g = np.random.default_rng(seed)
    parts = random_parts(fmt, group, n, k, g)
    qw = qweight_from_oracle(fmt, group, parts, n, k)
    x = g.standard_normal((1, k)).astype(np.float16)
    x[0, g.integers(0, k)] *= 50.0
    ldy = n + 4
    y = torch.full((ldy,), -1, dtype=torch.int16, device="cuda")
    say("ranges", fmt, group, "n", n, "k", k)
    rq.rq_gemm_small_m(dev_f16(x), 1, k, qw, y, ldy)
    torch.cuda.synchronize()
    out = host(y, np.float16, (1, ldy))
    assert np.all(out[:, n:].view(np.int16) == -1), "wrote past n"
    y_ref, b = ref.weight_only_ref(x, fmt, parts, group)
    ok, info = ref.compare(out[:, :n].astype(np.float64), y_ref, b)
    assert ok, info


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("n,k", SHAPES)
def test_ranges_m1(group, n, k):
    _run(quant.W4_SYM, group, n, k, n * 7 + k + group)


def test_ranges_fused_small():
    # three matrices of 200, 136 and 9 rows: 44 tiles of 8 in all
    k = 4096
    g = np.random.default_rng(5)
    ns = (200, 136, 9)
    parts = [random_parts(quant.W4_SYM, 64, n, k, g) for n in ns]
    qws = [qweight_from_oracle(quant.W4_SYM, 64, p, n, k) for p, n in zip(parts, ns)]
    xs = [g.standard_normal((1, k)).astype(np.float16) for _ in ns]
    ldy = 256
    ys = [torch.full((ldy,), -1, dtype=torch.int16, device="cuda") for _ in ns]
    say("ranges fused", ns, "k", k)
    rq.rq_fused_rkv(dev_f16(xs[0]), dev_f16(xs[1]), dev_f16(xs[2]), 1, k, *qws, *ys, ldy)
    torch.cuda.synchronize()
    for x, p, n, yv in zip(xs, parts, ns, ys):
        out = host(yv, np.float16, (1, ldy))
        assert np.all(out[:, n:].view(np.int16) == -1), "wrote past n"
        y_ref, b = ref.weight_only_ref(x, quant.W4_SYM, p, 64)
        ok, info = ref.compare(out[:, :n].astype(np.float64), y_ref, b)
        assert ok, (n, info)
