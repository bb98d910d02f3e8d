"""Decode chain (rq_chain_*): every product of a chained decode step against
the oracle.

A chain op's input is the fp16 output of an earlier op as the GPU wrote it,
so each op is checked on its own: y_q against the oracle's fp64
dequantize-then-multiply of x_q = (GPU's y_src), to the products' tolerance.
Weights are seeded symmetric int4 group-64 codes with fp16 scales chosen so
that outputs keep the input's scale (W ~ N(0, 1/K) in distribution), and an
fp16 head; the oracle reads the same bytes (every byte is a valid code).
"""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import dev_bytes, dev_f16, host, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu


def _w4_parts(n, k, g):
    # symmetric codes q in -7..7 (nibbles 1..15), as the quantizer makes them:
    # zero mean, so a long chain neither drifts nor overflows
    lo = g.integers(1, 16, (n, k // 2), dtype=np.uint8)
    hi = g.integers(1, 16, (n, k // 2), dtype=np.uint8)
    codes = (lo | (hi << 4)).astype(np.uint8)
    # rms of q is ~4.32: scales put the weights' rms near 1/sqrt(k)
    s = (g.uniform(0.75, 1.25, (n, k // 64)) / (4.32 * np.sqrt(k))).astype(np.float16)
    return {"codes": codes, "scales": s}


def _f16_parts(n, k, g):
    return {"codes": (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float16)}


def layer_ops(c, layers, vocab, order=("r", "k", "v")):
    """(name, fmt, n, k, src) of a chained decode step: per layer R/K/V (input:
    the previous layer's channel-mix value output, or the external x), O (input
    R), channel-mix key (input O) and value (input key); then the fp16 head."""
    ops = []
    prev = -1
    for layer in range(layers):
        base = len(ops)
        idx = {}
        for i, name in enumerate(order):
            idx[name] = base + i
            ops.append(("%s%d" % (name, layer), "w4", c, c, prev))
        o = len(ops)
        ops.append(("o%d" % layer, "w4", c, c, idx["r"]))
        ops.append(("key%d" % layer, "w4", 4 * c, c, o))
        ops.append(("value%d" % layer, "w4", c, 4 * c, o + 1))
        prev = o + 2
    if vocab:
        ops.append(("head", "f16", vocab, c, prev))
    return ops


class HostChain:
    """Weights and buffers of a chain, the GPU plan, and the oracle check."""

    def __init__(self, spec, seed):
        g = np.random.default_rng(seed)
        self.spec = spec
        self.parts, self.qw, self.y = [], [], []
        for name, fmt, n, k, src in spec:
            p = _w4_parts(n, k, g) if fmt == "w4" else _f16_parts(n, k, g)
            self.parts.append(p)
            if fmt == "w4":
                self.qw.append(rq.QWeight(rq.RQ_W4_SYM, 64, n, k, dev_bytes(p["codes"]), dev_bytes(p["scales"])))
            else:
                self.qw.append(rq.QWeight(rq.RQ_F16, 0, n, k, dev_bytes(p["codes"])))
            self.y.append(torch.zeros(n, dtype=torch.int16, device="cuda"))
        k0 = spec[0][3]
        self.x = g.standard_normal(k0).astype(np.float16)
        self.xd = dev_f16(self.x)
        ops = []
        for i, (name, fmt, n, k, src) in enumerate(spec):
            ops.append((self.qw[i], src, self.xd if src < 0 else None, self.y[i]))
        self.chain = rq.Chain(ops)

    def outputs(self):
        return [host(y, np.float16).copy() for y in self.y]

    def check(self, outs, rows=None):
        worst = 0.0
        for i, (name, fmt, n, k, src) in enumerate(self.spec):
            x = self.x if src < 0 else outs[src]
            assert np.all(np.isfinite(x)), name
            p = self.parts[i]
            sel = np.arange(n) if rows is None else rows[i]
            if fmt == "w4":
                what = quant.dequant(quant.W4_SYM, {"codes": p["codes"][sel], "scales": p["scales"][sel]}, 64)
            else:
                what = p["codes"][sel].astype(np.float64)
            y_ref, b = ref.matmul_ref(x.astype(np.float64)[None, :], what)
            ok, info = ref.compare(outs[i][sel][None, :], y_ref, b)
            assert ok, (name, self.chain.grid(i), info)
            worst = max(worst, info["max_ratio"])
        return worst


def test_chain_one_product():
    spec = [("r0", "w4", 2048, 2048, -1)]
    say("chain: one product 2048 x 2048")
    hc = HostChain(spec, 11)
    print("grids", [hc.chain.grid(i) for i in range(len(spec))], flush=True)
    hc.chain.run()
    hc.chain.check()
    hc.check(hc.outputs())
    hc.chain.destroy()


def test_chain_two_products():
    spec = [("r0", "w4", 2048, 2048, -1), ("o0", "w4", 2048, 2048, 0)]
    say("chain: two dependent products 2048 x 2048")
    hc = HostChain(spec, 12)
    hc.chain.run()
    hc.chain.check()
    hc.check(hc.outputs())
    hc.chain.destroy()


def test_chain_two_layers_width_2048():
    spec = layer_ops(2048, 2, 8192)
    say("chain width 2048, 2 layers + head 8192, %d ops" % len(spec))
    hc = HostChain(spec, 1)
    print("grids", [hc.chain.grid(i) for i in range(len(spec))], flush=True)
    hc.chain.run()
    torch.cuda.synchronize()
    hc.chain.check()
    outs = hc.outputs()
    worst = hc.check(outs)
    print("worst max_ratio %.3f" % worst, flush=True)
    # a second run is bit-identical (fixed reduction order)
    hc.chain.run()
    hc.chain.check()
    outs2 = hc.outputs()
    for a, b in zip(outs, outs2):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    hc.chain.destroy()


def test_chain_order_kvr_and_external_input_split():
    # R last among the three, so O waits on the product just before it; the
    # first three ops read the caller's x in K slices
    spec = layer_ops(2048, 1, 0, order=("k", "v", "r"))
    say("chain width 2048, order k v r, %d ops" % len(spec))
    hc = HostChain(spec, 2)
    hc.chain.run()
    hc.chain.check()
    hc.check(hc.outputs())
    hc.chain.destroy()


def test_chain_small_unsplit_shapes():
    # width 384: k = 3 chunks, so every product runs unsplit on a few workgroups
    spec = layer_ops(384, 2, 512)
    say("chain width 384, 2 layers + head 512")
    hc = HostChain(spec, 3)
    print("grids", [hc.chain.grid(i) for i in range(len(spec))], flush=True)
    hc.chain.run()
    hc.chain.check()
    hc.check(hc.outputs())
    hc.chain.destroy()


def test_chain_graph_replays():
    spec = layer_ops(2048, 1, 4096)
    say("chain graph replays, width 2048")
    hc = HostChain(spec, 4)
    hc.chain.run()
    hc.chain.check()
    eager = hc.outputs()
    hc.check(eager)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            hc.chain.run(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in hc.y:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hc.chain.check()
        got = hc.outputs()
        for a, b in zip(eager, got):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), rep
        hc.chain.run()  # eager work between replays
        torch.cuda.synchronize()
    del g
    hc.chain.destroy()


def test_chain_width_4096_sampled_rows():
    # the 13.3B shapes (two layers) and the 65536 x 4096 head, sampled rows
    spec = layer_ops(4096, 2, 65536)
    say("chain width 4096, 2 layers + head 65536 (sampled rows)")
    hc = HostChain(spec, 5)
    print("grids", [hc.chain.grid(i) for i in range(len(spec))], flush=True)
    hc.chain.run()
    hc.chain.check()
    outs = hc.outputs()
    g = np.random.default_rng(7)
    rows = []
    for name, fmt, n, k, src in spec:
        pick = g.choice(n, size=64, replace=False)
        rows.append(np.sort(np.concatenate([pick, [0, n - 1]])))
    hc.check(outs, rows)
    hc.chain.destroy()
