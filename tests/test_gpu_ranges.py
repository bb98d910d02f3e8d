"""int4 products at M <= 8 on matrices of fewer than 256 row tiles of 16,
where each 8-row tile covers K as two halves (the MFMA's diagonal blocks,
A row h M + m against column h 8 + r): tile counts from one to 255, ragged
last tiles (n not a multiple of 8 or 16), halves of 16 to 64 chunks with
ragged waves, both int4 groups, activation and output strides wider than
K and n, fused R/K/V with three small matrices, and the neighbours that take
other plans (M = 9; K of fewer than 32 chunks or a chunk count that is not a
multiple of eight).  Outputs are compared with the oracle on every row of
the small matrices and on sampled rows (always the last nine) of the large
ones; the bytes after n must stay untouched."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_f16, host, qweight_from_oracle, random_parts, rows_of, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu

# two halves from 32 chunks (K = 4096) when the chunk count is a multiple of
# eight; (2048, 2048) and (300, 1536) take other plans
SHAPES = [(2048, 8192), (1000, 4096), (8, 4096), (9, 5120), (136, 5120), (4072, 4096), (2040, 16384),
          (2048, 2048), (300, 1536)]
MS = [1, 2, 3, 5, 8, 9]

_cache = {}


def _weight(group, n, k):
    key = (group, n, k)
    if key not in _cache:
        _cache.clear()
        g = np.random.default_rng(n * 7 + k + group)
        parts = random_parts(quant.W4_SYM, group, n, k, g)
        _cache[key] = (parts, qweight_from_oracle(quant.W4_SYM, group, parts, n, k))
    return _cache[key]


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", MS)
def test_ranges(group, n, k, m):
    parts, qw = _weight(group, n, k)
    g = np.random.default_rng(m * 1000 + n + k)
    ldx = k + 8 * (m % 3)
    x = g.standard_normal((m, ldx)).astype(np.float16)
    x[:, g.integers(0, k)] *= 50.0
    ldy = n + 4
    y = torch.full((m * ldy,), -1, dtype=torch.int16, device="cuda")
    say("ranges", group, "n", n, "k", k, "m", m)
    rq.rq_gemm_small_m(dev_f16(x), m, ldx, qw, y, ldy)
    torch.cuda.synchronize()
    out = host(y, np.float16, (m, ldy))
    assert np.all(out[:, n:].view(np.int16) == -1), "wrote past n"
    if n > 1100:
        rows = np.concatenate([np.sort(g.choice(n - 9, 55, replace=False)), np.arange(n - 9, n)])
        sub = rows_of(parts, rows)
    else:
        rows, sub = np.arange(n), parts
    y_ref, b = ref.weight_only_ref(x[:, :k], quant.W4_SYM, sub, group)
    ok, info = ref.compare(out[:, rows].astype(np.float64), y_ref, b)
    assert ok, info


@pytest.mark.parametrize("m", [1, 4, 8])
def test_ranges_fused_small(m):
    # three matrices of 200, 136 and 9 rows: 44 tiles of 8 in all
    k = 4096
    g = np.random.default_rng(5 + m)
    ns = (200, 136, 9)
    parts = [random_parts(quant.W4_SYM, 64, n, k, g) for n in ns]
    qws = [qweight_from_oracle(quant.W4_SYM, 64, p, n, k) for p, n in zip(parts, ns)]
    xs = [g.standard_normal((m, k)).astype(np.float16) for _ in ns]
    ldy = 256
    ys = [torch.full((m * ldy,), -1, dtype=torch.int16, device="cuda") for _ in ns]
    say("ranges fused", ns, "k", k, "m", m)
    rq.rq_fused_rkv(dev_f16(xs[0]), dev_f16(xs[1]), dev_f16(xs[2]), m, k, *qws, *ys, ldy)
    torch.cuda.synchronize()
    for x, p, n, yv in zip(xs, parts, ns, ys):
        out = host(yv, np.float16, (m, ldy))
        assert np.all(out[:, n:].view(np.int16) == -1), "wrote past n"
        y_ref, b = ref.weight_only_ref(x, quant.W4_SYM, p, 64)
        ok, info = ref.compare(out[:, :n].astype(np.float64), y_ref, b)
        assert ok, (n, info)


SB_SHAPES = [(2560, 10240), (1000, 4096), (9, 5120), (136, 4096), (2560, 2560)]


@pytest.mark.parametrize("n,k", SB_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9])
def test_ranges_sb256(n, k, m):
    # superblock codes at the same shapes keep their one-range plans (unsplit,
    # or four K slices on fewer than 256 row tiles at M <= 4): the planner's
    # boundary between the formats
    g = np.random.default_rng(n + k + m)
    key = ("sb", n, k)
    if key not in _cache:
        _cache.clear()
        parts = random_parts(quant.W4_ASYM_SB256, 32, n, k, g)
        _cache[key] = (parts, qweight_from_oracle(quant.W4_ASYM_SB256, 32, parts, n, k))
    parts, qw = _cache[key]
    ldx = k + 8 * (m % 3)
    x = g.standard_normal((m, ldx)).astype(np.float16)
    x[:, g.integers(0, k, 4)] *= 50.0
    ldy = n + 4
    y = torch.full((m * ldy,), -1, dtype=torch.int16, device="cuda")
    say("ranges sb256", "n", n, "k", k, "m", m)
    rq.rq_gemm_small_m(dev_f16(x), m, ldx, qw, y, ldy)
    torch.cuda.synchronize()
    out = host(y, np.float16, (m, ldy))
    assert np.all(out[:, n:].view(np.int16) == -1), "wrote past n"
    if n > 1100:
        rows = np.concatenate([np.sort(g.choice(n - 9, 55, replace=False)), np.arange(n - 9, n)])
        sub = rows_of(parts, rows)
    else:
        rows, sub = np.arange(n), parts
    y_ref, b = ref.weight_only_ref(x[:, :k], quant.W4_ASYM_SB256, sub, 32)
    ok, info = ref.compare(out[:, rows].astype(np.float64), y_ref, b)
    assert ok, info
