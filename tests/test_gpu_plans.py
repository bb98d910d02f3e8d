"""Every weight format of the small-M products across the batch sizes where
the launch planner changes shape: one or two activation tiles, unsplit
slices in LDS (small and large), K split over workspace slices with shared
row tiles, per-wave streamed activations, and waves of 2 to 16 chunks.

Shapes are large enough to reach those plans (131 and 194 row tiles, the
last one partial) and have ragged chunk counts (the last wave of a slice
holds fewer valid chunks than it owns), int8 group 64 with an odd number of
scales per row.  Codes, scales and weights are seeded random inputs; the
oracle multiplies sampled rows, including the last five."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_f16, host, qweight_from_oracle, random_parts, rows_of, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu

# (format, group, k): k ragged in the format's chunk (128 k for 4-, 5-, 6-bit
# codes, 64 for int8, 32 for fp16 / bf16); int4 group 16 runs the first kernel
FORMATS = [(quant.W4_SYM, 64, 128 * 67), (quant.W4_SYM, 32, 128 * 45), (quant.W4_SYM, 16, 128 * 33),
           (quant.W8_SYM, 64, 64 * 131), (quant.W8_SYM, 32, 64 * 75), (quant.W8_SYM, 16, 64 * 41),
           (quant.W4_ASYM_SB256, 32, 256 * 35), (quant.F16, 0, 32 * 133), (quant.BF16, 0, 32 * 99),
           (quant.W6_SYM, 32, 128 * 41), (quant.W5_SYM, 64, 128 * 53)]
MS = [1, 2, 3, 5, 8, 12, 16, 17, 25, 32]

_cache = {}


def _weight(fmt, group, n, k):
    key = (fmt, group, n, k)
    if key not in _cache:
        _cache.clear()                      # one weight on the device at a time
        g = np.random.default_rng(n * 31 + k + fmt)
        parts = random_parts(fmt, group, n, k, g)
        _cache[key] = (parts, qweight_from_oracle(fmt, group, parts, n, k))
    return _cache[key]


def _check(fmt, group, n, k, m, ws=None):
    parts, qw = _weight(fmt, group, n, k)
    g = np.random.default_rng(m * 1000 + k)
    ldx = k + 8 * (m % 3)
    x = g.standard_normal((m, ldx)).astype(np.float16)
    ldy = n + 4
    y = torch.full((m * ldy,), -1, dtype=torch.int16, device="cuda")
    say("plans", fmt, group, "n", n, "k", k, "m", m, "ws", ws)
    rq.rq_gemm_small_m(dev_f16(x), m, ldx, qw, y, ldy, ws=ws)
    torch.cuda.synchronize()
    out = host(y, np.float16, (m, ldy))
    assert np.all(out[:, n:].view(np.int16) == -1), "wrote past n"
    rows = np.concatenate([np.sort(g.choice(n - 5, 27, replace=False)), np.arange(n - 5, n)])
    y_ref, b = ref.weight_only_ref(x[:, :k], fmt, rows_of(parts, rows), group)
    ok, info = ref.compare(out[:, rows].astype(np.float64), y_ref, b)
    assert ok, (m, info)


@pytest.mark.parametrize("fmt,group,k", FORMATS)
@pytest.mark.parametrize("m", MS)
def test_plans_131_tiles(fmt, group, k, m):
    _check(fmt, group, 2085, k, m)


@pytest.mark.parametrize("fmt,group,k", [f for f in FORMATS if f[0] in (quant.W4_SYM, quant.W4_ASYM_SB256,
                                                                       quant.W6_SYM, quant.W5_SYM) and f[1] != 16])
@pytest.mark.parametrize("m", [4, 8, 17, 32])
def test_plans_194_tiles(fmt, group, k, m):
    # 194 row tiles: the per-wave streamed plan wherever the slice is too
    # large for LDS (two tiles from M = 17, one tile from M = 4 at the
    # larger K)
    _check(fmt, group, 3100, 2 * k if k < 8192 else k, m)


@pytest.mark.parametrize("fmt,group", [(quant.W5_SYM, 32), (quant.W6_SYM, 32), (quant.W4_ASYM_SB256, 32),
                                       (quant.W8_SYM, 16)])
@pytest.mark.parametrize("n,k,m", [(10240, 2560, 9), (10240, 2560, 16), (2560, 10240, 1), (2560, 10240, 4),
                                   (2560, 10240, 16), (7680, 2560, 16)])
def test_plans_2p9b_shapes(fmt, group, n, k, m):
    # the 2.9B-width channel-mix shapes and three stacked projections: at
    # M = 9..16 the key's 640 row tiles would need two rounds of one
    # workgroup per CU unsplit, so K is split
    _check(fmt, group, n, k, m)


@pytest.mark.parametrize("fmt,group", [(quant.W4_ASYM_SB256, 32), (quant.W4_SYM, 32), (quant.W6_SYM, 32),
                                       (quant.W5_SYM, 64), (quant.W4_SYM, 64)])
@pytest.mark.parametrize("k,m", [(8192, 32), (8192, 20), (16384, 4), (16384, 8)])
def test_streamed_without_workspace(fmt, group, k, m):
    """Without a workspace no K split is possible, and 194 row tiles with an
    activation slice too large for LDS take the per-wave streamed plan for
    every format (with a workspace, one activation tile and SB256 split K
    instead)."""
    n = 3100
    plan = rq.rq_plan_small_m((fmt, 32 if fmt == quant.W4_ASYM_SB256 else group, n, k), m, ldx=k + 8 * (m % 3),
                              ws_bytes=0)
    assert plan["kernel"] == rq.RQ_PLAN_STREAMED_X, plan
    _check(fmt, group, n, k, m, ws=False)
