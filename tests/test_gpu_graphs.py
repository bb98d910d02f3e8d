"""Products captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each replay runs after eager work of the program's own (the outputs are
cleared and the same products run eagerly on the default stream) and a
synchronization, and must reproduce the eager results bit for bit: a launch
shape is a function of the call's arguments alone, workspace included, so the
graph holds the eager calls' shapes whether or not the capture stream ever ran
a product before.  Products given no workspace take unsplit launch shapes;
their graph must match eager calls without a workspace bit for bit, and the
oracle within its tolerance.
"""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_f16, host, qweight_from_oracle, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu


def _w(n, k, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)


def _x(m, k, seed):
    return np.random.default_rng(seed).standard_normal((m, k)).astype(np.float16)


# (format, group, n, k, m): split-K (2048x8192 at M = 32), streamed (4000x4096
# at M = 32), unsplit, 6-bit, bf16, and SB256
CASES = [(quant.W4_SYM, 64, 2048, 8192, 32), (quant.W4_SYM, 64, 4000, 4096, 32), (quant.W4_SYM, 64, 512, 2048, 1),
         (quant.W4_SYM, 64, 2048, 2048, 8), (quant.W6_SYM, 32, 768, 1024, 5), (quant.BF16, 0, 640, 1024, 3),
         (quant.W4_ASYM_SB256, 32, 1024, 2560, 16), (quant.W8_SYM, 16, 300, 768, 2)]


def _setup():
    items = []
    for i, (fmt, group, n, k, m) in enumerate(CASES):
        w = _w(n, k, 100 + i)
        parts = quant.quantize(w, fmt, group)
        qw = qweight_from_oracle(fmt, group, parts, n, k)
        x = _x(m, k, 200 + i)
        items.append({"fmt": fmt, "group": group, "n": n, "k": k, "m": m, "parts": parts, "qw": qw, "x": x,
                      "xd": dev_f16(x), "y": torch.zeros(m * n, dtype=torch.int16, device="cuda")})
    return items


def _run(items, ws=None):
    for it in items:
        rq.rq_gemm_small_m(it["xd"], it["m"], it["k"], it["qw"], it["y"], it["n"], ws=ws)


def test_graph_replays_match_eager():
    items = _setup()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("graph: eager warm-up on the capture stream")
    with torch.cuda.stream(s):
        _run(items)
    torch.cuda.synchronize()
    eager = [it["y"].clone() for it in items]
    for it, e in zip(items, eager):
        y_ref, b = ref.weight_only_ref(it["x"], it["fmt"], it["parts"], it["group"])
        ok, info = ref.compare(host(e, np.float16, (it["m"], it["n"])).astype(np.float64), y_ref, b)
        assert ok, (it["fmt"], it["n"], it["k"], it["m"], info)
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g, stream=s):
        _run(items)
    torch.cuda.synchronize()
    for rep in range(4):
        for it in items:
            it["y"].zero_()
        _run(items)                      # eager work of the program's own, on the default stream
        torch.cuda.synchronize()
        for it in items:
            it["y"].fill_(-1)
        torch.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for it, e in zip(items, eager):
            assert torch.equal(it["y"], e), (rep, it["fmt"], it["n"], it["k"], it["m"])


def test_graph_without_warmup_is_bit_identical():
    """A graph captured on a stream that never ran a product eagerly holds the
    same launch shapes, and gives the same bits, as eager calls with the same
    workspace on another stream."""
    items = _setup()
    rq.default_workspace()
    _run(items)                          # eager, default stream
    torch.cuda.synchronize()
    eager = [it["y"].clone() for it in items]
    s = torch.cuda.Stream()              # no product has run on it
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    say("graph: capture with no warm-up on the capture stream")
    with torch.cuda.graph(g, stream=s):
        _run(items)
    for rep in range(3):
        for it in items:
            it["y"].fill_(-1)
        torch.cuda.synchronize()
        say("graph: replay with no warm-up", rep)
        g.replay()
        torch.cuda.synchronize()
        for it, e in zip(items, eager):
            assert torch.equal(it["y"], e), (rep, it["fmt"], it["n"], it["k"], it["m"])


def test_graph_without_workspace():
    items = [it for it in _setup() if it["fmt"] in (quant.W4_SYM, quant.W8_SYM, quant.W4_ASYM_SB256)]
    _run(items, ws=False)
    torch.cuda.synchronize()
    eager = [it["y"].clone() for it in items]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    say("graph: capture without workspace")
    with torch.cuda.graph(g, stream=s):
        _run(items, ws=False)
    for rep in range(3):
        for it in items:
            it["y"].fill_(-1)
        torch.cuda.synchronize()
        say("graph: replay without workspace", rep)
        g.replay()
        torch.cuda.synchronize()
        for it, e in zip(items, eager):
            assert torch.equal(it["y"], e), (rep, it["fmt"], it["n"], it["k"], it["m"])
            y_ref, b = ref.weight_only_ref(it["x"], it["fmt"], it["parts"], it["group"])
            ok, info = ref.compare(host(it["y"], np.float16, (it["m"], it["n"])).astype(np.float64), y_ref, b)
            assert ok, (rep, it["fmt"], it["n"], it["k"], it["m"], info)


def test_graph_gemm_w4_and_fused_rkv():
    """The int4 prefill GEMM (split K through the workspace at this shape) and
    the fused R/K/V call, captured together and replayed."""
    n, k, m = 1024, 4096, 64
    parts = quant.quantize(_w(n, k, 7), quant.W4_SYM, 64)
    qw = qweight_from_oracle(quant.W4_SYM, 64, parts, n, k)
    x = _x(m, k, 8)
    xd = dev_f16(x)
    y = torch.zeros(m * n, dtype=torch.int16, device="cuda")
    c, mr = 768, 4
    rp = [quant.quantize(_w(c, c, 20 + i), quant.W8_SYM, 64) for i in range(3)]
    rq3 = [qweight_from_oracle(quant.W8_SYM, 64, p, c, c) for p in rp]
    xr = _x(mr, c, 9)
    xrd = dev_f16(xr)
    ys = [torch.zeros(mr * c, dtype=torch.int16, device="cuda") for _ in range(3)]

    def run():
        rq.rq_gemm_w4(xd, m, k, qw, y, n)
        rq.rq_fused_rkv(xrd, xrd, xrd, mr, c, rq3[0], rq3[1], rq3[2], ys[0], ys[1], ys[2], c)

    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in [y] + ys]
    y_ref, b = ref.weight_only_ref(x, quant.W4_SYM, parts, 64)
    ok, info = ref.compare(host(eager[0], np.float16, (m, n)).astype(np.float64), y_ref, b)
    assert ok, info
    g = torch.cuda.CUDAGraph()
    say("graph: capture gemm_w4 + fused_rkv")
    with torch.cuda.graph(g, stream=s):
        run()
    for rep in range(3):
        run()                            # eager, default stream
        torch.cuda.synchronize()
        for t in [y] + ys:
            t.fill_(-1)
        torch.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip([y] + ys, eager):
            assert torch.equal(t, e), rep


def test_graph_replays_planner_shapes():
    """Launch shapes added to the planner, captured and replayed: a long K
    cut four ways for SB256 on 160 row tiles (M = 1), one-tile streamed
    activations (4-bit codes, 194 row tiles, M = 6), a split whose last
    slices are empty (6-bit, 41 chunks, M = 32) and the two-range 8-row
    tiles (int4, 128 and 63 row tiles of 16, M = 1 and 8)."""
    from gpu_helpers import random_parts
    cases = [(quant.W4_ASYM_SB256, 32, 2560, 10240, 1), (quant.W4_SYM, 32, 3100, 16384, 6),
             (quant.W6_SYM, 32, 2085, 5248, 32), (quant.W4_SYM, 64, 2048, 8192, 1),
             (quant.W4_SYM, 32, 1000, 4096, 8)]
    items = []
    for i, (fmt, group, n, k, m) in enumerate(cases):
        g = np.random.default_rng(300 + i)
        parts = random_parts(fmt, group, n, k, g)
        x = _x(m, k, 400 + i)
        items.append({"fmt": fmt, "group": group, "n": n, "k": k, "m": m, "parts": parts, "x": x,
                      "qw": qweight_from_oracle(fmt, group, parts, n, k), "xd": dev_f16(x),
                      "y": torch.zeros(m * n, dtype=torch.int16, device="cuda")})
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        _run(items)
    torch.cuda.synchronize()
    eager = [it["y"].clone() for it in items]
    g = torch.cuda.CUDAGraph()
    say("graph: capture planner shapes")
    with torch.cuda.graph(g, stream=s):
        _run(items)
    for rep in range(3):
        _run(items)                      # eager, default stream
        torch.cuda.synchronize()
        for it in items:
            it["y"].fill_(-1)
        torch.cuda.synchronize()
        say("graph: replay planner shapes", rep)
        g.replay()
        torch.cuda.synchronize()
        for it, e in zip(items, eager):
            assert torch.equal(it["y"], e), (rep, it["fmt"], it["n"], it["k"], it["m"])
    rows = np.arange(0, 2560, 97)
    it = items[0]
    y_ref, b = ref.weight_only_ref(it["x"], it["fmt"], {nm: a[rows] for nm, a in it["parts"].items()}, 32)
    ok, info = ref.compare(host(eager[0], np.float16, (1, 2560))[:, rows].astype(np.float64), y_ref, b)
    assert ok, info
