"""K-split weight-streaming products cut into up to four slices add their
partial tiles inside the same launch: the last workgroup of each tile group,
found through an arrival counter at the head of the workspace, sums the slices
in slice order (more slices go through a second, reducing kernel).

Checked here, on shapes whose plans split K in four: the phased kernel with
two activation tiles (two or four row tiles per workgroup, the latter on
sixteen waves, with ragged last tile groups) and with one
(M = 9..16, where the streaming kernel would need eight slices), the
streaming kernel at M = 16, the four-slice plans of SB256, int8 group 16 and
6-bit codes at M <= 4, ragged tile counts.  Every call leaves the counters at
zero; repeated calls, calls on a caller-owned zero-filled workspace and graph
replays give bit-identical outputs; a workspace with no room past the
counters means no split; and sampled rows agree with the oracle."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_f16, host, qweight_from_oracle, random_parts, rows_of, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 64 << 10

# (format, group, n, k, m)
SHAPES = [
    (quant.W4_SYM, 64, 2048, 8192, 32),       # phased, two tiles per workgroup, K in 4 slices
    (quant.W4_SYM, 64, 2085, 8192, 17),       # phased, ragged last tile group
    (quant.W4_SYM, 64, 4096, 16384, 16),      # phased with one activation tile, K in 4 slices
    (quant.W4_SYM, 64, 4096, 16384, 32),      # phased, K in 4 slices
    (quant.W4_SYM, 64, 2048, 8192, 16),       # streaming, K in 4 slices, shared tiles
    (quant.W4_SYM, 64, 4100, 16384, 12),      # phased with one activation tile, ragged last tile group
    (quant.W4_SYM, 64, 4100, 16384, 32),      # phased, sixteen waves on four row tiles, ragged last group
    (quant.W4_SYM, 64, 4100, 16384, 20),      # the same with activation rows 20..31 empty
    (quant.W4_SYM, 32, 4100, 8192, 24),       # group 32, four row tiles, ragged
    (quant.W4_SYM, 32, 4096, 16384, 9),
    (quant.W4_ASYM_SB256, 32, 2560, 10240, 1),  # four-slice plan of the costlier decoders
    (quant.W8_SYM, 16, 2560, 10240, 4),
    (quant.W6_SYM, 32, 1000, 10240, 3),
]

_cache = {}


def _weight(fmt, group, n, k):
    key = (fmt, group, n, k)
    if key not in _cache:
        _cache.clear()
        g = np.random.default_rng(n * 7 + k + fmt)
        parts = random_parts(fmt, group, n, k, g)
        _cache[key] = (parts, qweight_from_oracle(fmt, group, parts, n, k))
    return _cache[key]


def _counters_zero():
    ws = rq.default_workspace()
    return bool((ws[:COUNTER_BYTES] == 0).all())


@pytest.mark.parametrize("fmt,group,n,k,m", SHAPES)
def test_split_in_launch(fmt, group, n, k, m):
    parts, qw = _weight(fmt, group, n, k)
    plan = rq.rq_plan_small_m(qw, m, k)
    assert plan["split"] > 1, plan
    assert plan["workspace_bytes"] > COUNTER_BYTES
    g = np.random.default_rng(m + n)
    x = g.standard_normal((m, k)).astype(np.float16)
    xd = dev_f16(x)
    y = torch.empty(m * n, dtype=torch.int16, device="cuda")
    say("split", fmt, group, n, k, m, plan)
    assert _counters_zero()
    rq.rq_gemm_small_m(xd, m, k, qw, y, n)
    torch.cuda.synchronize()
    assert _counters_zero(), "a call left a split counter non-zero"
    first = y.clone()
    out = host(y, np.float16, (m, n))
    rows = np.concatenate([np.sort(g.choice(n - 3, 29, replace=False)), np.arange(n - 3, n)])
    y_ref, b = ref.weight_only_ref(x, fmt, rows_of(parts, rows), group)
    ok, info = ref.compare(out[:, rows].astype(np.float64), y_ref, b)
    assert ok, info
    # again, then on a caller-owned zero-filled workspace on a side stream
    for _ in range(3):
        rq.rq_gemm_small_m(xd, m, k, qw, y, n)
    torch.cuda.synchronize()
    assert torch.equal(y, first)
    own = torch.zeros(rq.rq_workspace_bytes(), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()    # the zero fill ran on the current stream
    st = torch.cuda.Stream()
    y2 = torch.empty_like(y)
    with torch.cuda.stream(st):
        rq.rq_gemm_small_m(xd, m, k, qw, y2, n, ws=own)
        rq.rq_gemm_small_m(xd, m, k, qw, y2, n, ws=own)
    torch.cuda.synchronize()
    assert torch.equal(y2, first)
    assert bool((own[:COUNTER_BYTES] == 0).all())
    del own


def test_no_room_past_counters_means_no_split():
    fmt, group, n, k, m = SHAPES[0]
    parts, qw = _weight(fmt, group, n, k)
    assert rq.rq_plan_small_m(qw, m, k, ws_bytes=COUNTER_BYTES)["split"] == 1
    assert rq.rq_plan_small_m(qw, m, k, ws_bytes=COUNTER_BYTES)["workspace_bytes"] == 0
    g = np.random.default_rng(5)
    x = g.standard_normal((m, k)).astype(np.float16)
    small = torch.zeros(COUNTER_BYTES, dtype=torch.uint8, device="cuda")
    y = torch.empty(m * n, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    say("split: 64 KiB workspace", n, k, m)
    rq.rq_gemm_small_m(dev_f16(x), m, k, qw, y, n, ws=small)
    torch.cuda.synchronize()
    assert bool((small == 0).all()), "an unsplit launch wrote the workspace"
    rows = np.arange(0, n, 97)
    y_ref, b = ref.weight_only_ref(x, fmt, rows_of(parts, rows), group)
    ok, info = ref.compare(host(y, np.float16, (m, n))[:, rows].astype(np.float64), y_ref, b)
    assert ok, info


def test_split_graph_replays():
    """Several split products in one graph, replayed with eager split calls
    between the replays: every replay equals the eager result and the
    counters are zero after each."""
    items = []
    for fmt, group, n, k, m in SHAPES[:4]:
        parts, qw = _weight(fmt, group, n, k)
        _cache.clear()
        g = np.random.default_rng(n + 3 * m)
        x = dev_f16(g.standard_normal((m, k)).astype(np.float16))
        items.append((qw, x, m, k, n, torch.empty(m * n, dtype=torch.int16, device="cuda")))
    rq.default_workspace()

    def run(outs):
        for (qw, x, m, k, n, _), y in zip(items, outs):
            rq.rq_gemm_small_m(x, m, k, qw, y, n)

    eager = [it[5] for it in items]
    say("split graph: eager")
    run(eager)
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    say("split graph: capture")
    with torch.cuda.graph(gr, stream=s):
        run(outs)
    for rep in range(4):
        for o in outs:
            o.fill_(-1)
        say("split graph: replay", rep)
        gr.replay()
        torch.cuda.synchronize()
        assert _counters_zero()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), rep
        run([torch.empty_like(e) for e in eager])   # eager split calls between the replays
        torch.cuda.synchronize()
