"""Benchmark of the quantized-weight decode and prefill products on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = the width-2048 (RWKV-7 1.5B) layer of symmetric int4 group-64
projections (fused R/K/V, O, cmix key, cmix value), fp16 activations with
channel 1202 scaled x50, decoded at each batch M in {1, 8, 32}, followed by
the width-4096 (7.2B) prefill set (per-token fp8 activation quantization, then
R, K, V, O, cmix key and cmix value as fp8 e4m3 per-channel GEMMs) at M = 256.
Every pass is a captured HIP graph over rotated copies of the weights (more
than 1 GiB in each rotation, so the 256 MB last-level cache cannot hold them);
inputs are resident in HBM before timing.

value = packed weight bytes streamed by the decode passes / their time (GB/s).
The JSON line also carries the fp8 prefill rate, the roofline of the dominant
kernel (the kernel class with the largest share of a step's time, its
average launch duration measured with HIP events around back-to-back
launches on the launching stream), and the CPU oracle on a bounded sample.

Synthetic weights: N(0, 1/K) from a seeded generator on the GPU, quantized
with rq_quantize_rtn.  --kernel-only runs just the dominant kernel's launch
loop and a calibration copy (for hardware-counter runs).
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gemm_rwkv_amd.rq as rq  # noqa: E402
from gemm_rwkv_amd import presets, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
F16_PEAK_TFLOPS = 2500.0
METRIC = "weight-stream GB/s (% HBM peak) W4g64 GEMV M=1..32; TFLOPS fp8 GEMM M=256"
ROTATE_BYTES = 1 << 30
C1, MS = 2048, (1, 8, 32)   # decode layer width, batches
C3, M3 = 4096, 256          # prefill width, batch
CALIB_BYTES = 256 << 20     # calibration copy for the traffic counters


def f16_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).view(np.int16)).to(dev)


_CAPTURE_STREAM = None


def capture(fn):
    """Graph of fn's launches.  An eager run goes first on the capture stream:
    it loads the code objects and allocates the binding's default workspace,
    which the graph's products then share."""
    global _CAPTURE_STREAM
    if _CAPTURE_STREAM is None:
        _CAPTURE_STREAM = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(_CAPTURE_STREAM):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=_CAPTURE_STREAM):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps, warmup=2, launches=1):
    """Median ms per replay over at least `reps` replays and at least 200
    dispatches (`launches` per replay); HIP events on the current stream,
    where the graph runs, around each replay."""
    reps = max(reps, -(-200 // max(launches, 1)))
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))


class Decode:
    """Rotated copies of the width-C int4 g64 layer and the decode launches."""

    def __init__(self, c, gen, dev):
        self.c = c
        shapes = synth.layer_shapes(c)
        per_set = sum(rq.rq_qweight_bytes(rq.RQ_W4_SYM, 64, n, k)[0] + rq.rq_qweight_bytes(rq.RQ_W4_SYM, 64, n, k)[1]
                      for _, n, k in shapes)
        self.copies = -(-ROTATE_BYTES // per_set)
        self.sets = []
        for _ in range(self.copies):
            s = {}
            for mat, n, k in shapes:
                wf = torch.randn(n, k, generator=gen, device=dev, dtype=torch.float32) * (1.0 / k ** 0.5)
                s[mat] = rq.quantize(wf, rq.RQ_W4_SYM, 64)
                del wf
            self.sets.append(s)
        self.set_bytes = per_set
        self.x = {m: f16_dev(synth.act_channel_1202(m, c), dev) for m in MS}
        self.x4 = {m: f16_dev(synth.act_normal(m, 4 * c, 1), dev) for m in MS}
        self.y = {m: {nm: torch.empty(m * (4 * c if nm == "key" else c), dtype=torch.int16, device=dev)
                      for nm in ("r", "k", "v", "o", "key", "val")} for m in MS}

    def rkv(self, s, m):
        y = self.y[m]
        rq.rq_fused_rkv(self.x[m], self.x[m], self.x[m], m, self.c, s[synth.MAT_R], s[synth.MAT_K],
                        s[synth.MAT_V], y["r"], y["k"], y["v"], self.c)

    def o(self, s, m):
        rq.rq_gemm_small_m(self.x[m], m, self.c, s[synth.MAT_O], self.y[m]["o"], self.c)

    def key(self, s, m):
        rq.rq_gemm_small_m(self.x[m], m, self.c, s[synth.MAT_KEY], self.y[m]["key"], 4 * self.c)

    def value(self, s, m):
        rq.rq_gemm_small_m(self.x4[m], m, 4 * self.c, s[synth.MAT_VALUE], self.y[m]["val"], self.c)

    def passes(self, m):
        for s in self.sets:
            self.rkv(s, m)
            self.o(s, m)
            self.key(s, m)
            self.value(s, m)

    def classes(self, m):
        """(name, launch-one(s), weight bytes per launch, launches per step)."""
        c = self.c
        b = lambda n, k: sum(rq.rq_qweight_bytes(rq.RQ_W4_SYM, 64, n, k)[:2])  # noqa: E731
        return [
            ("gemv w4g64 fused R/K/V 3x%dx%d M=%d" % (c, c, m), lambda s: self.rkv(s, m), 3 * b(c, c), self.copies),
            ("gemv w4g64 O %dx%d M=%d" % (c, c, m), lambda s: self.o(s, m), b(c, c), self.copies),
            ("gemv w4g64 cmix key %dx%d M=%d" % (4 * c, c, m), lambda s: self.key(s, m), b(4 * c, c), self.copies),
            ("gemv w4g64 cmix value %dx%d M=%d" % (c, 4 * c, m), lambda s: self.value(s, m), b(c, 4 * c),
             self.copies),
        ]


class Prefill:
    """Rotated copies of the width-C fp8 per-channel set and the M=256 prefill launches."""

    def __init__(self, c, m, gen, dev):
        self.c, self.m = c, m
        shapes = synth.layer_shapes(c)
        per_set = sum(n * k + 4 * n for _, n, k in shapes)
        self.copies = -(-ROTATE_BYTES // per_set)
        self.sets = []
        for _ in range(self.copies):
            s = {}
            for mat, n, k in shapes:
                wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
                s[mat] = rq.quantize(wf, rq.RQ_FP8_E4M3_CH)
                del wf
            self.sets.append(s)
        self.set_bytes = per_set
        self.flops = sum(2.0 * m * n * k for _, n, k in shapes)
        self.xa = f16_dev(synth.act_normal(m, c, 3), dev)
        self.xa4 = f16_dev(synth.act_normal(m, 4 * c, 3, salt=1), dev)
        self.xq = torch.empty(m * c, dtype=torch.uint8, device=dev)
        self.xq4 = torch.empty(m * 4 * c, dtype=torch.uint8, device=dev)
        self.sx = torch.empty(m, dtype=torch.float32, device=dev)
        self.sx4 = torch.empty(m, dtype=torch.float32, device=dev)
        self.y = torch.empty(m * 4 * c, dtype=torch.int16, device=dev)

    def aq(self, _s=None):
        rq.rq_quantize_act(self.xa, self.m, self.c, self.c, rq.RQ_FP8_E4M3_CH, self.xq, self.sx)

    def aq4(self, _s=None):
        rq.rq_quantize_act(self.xa4, self.m, 4 * self.c, 4 * self.c, rq.RQ_FP8_E4M3_CH, self.xq4, self.sx4)

    def gemm(self, s, mat):
        w = s[mat]
        if mat == synth.MAT_VALUE:
            rq.rq_gemm_fp8(self.xq4, self.sx4, self.m, w, self.y, w.n)
        else:
            rq.rq_gemm_fp8(self.xq, self.sx, self.m, w, self.y, w.n)

    def passes(self):
        for s in self.sets:
            self.aq()
            for mat in (synth.MAT_R, synth.MAT_K, synth.MAT_V, synth.MAT_O, synth.MAT_KEY):
                self.gemm(s, mat)
            self.aq4()
            self.gemm(s, synth.MAT_VALUE)

    def classes(self):
        c, m = self.c, self.m
        fl = lambda n, k: 2.0 * m * n * k  # noqa: E731
        return [
            ("fp8 act quant %dx%d" % (m, c), self.aq, 0, self.copies, 0.0),
            ("fp8 act quant %dx%d" % (m, 4 * c), self.aq4, 0, self.copies, 0.0),
            ("gemm fp8 %dx%dx%d (R,K,V,O)" % (m, c, c), lambda s: self.gemm(s, synth.MAT_R),
             c * c + 4 * c, 4 * self.copies, fl(c, c)),
            ("gemm fp8 %dx%dx%d (cmix key)" % (m, 4 * c, c), lambda s: self.gemm(s, synth.MAT_KEY),
             4 * c * c + 16 * c, self.copies, fl(4 * c, c)),
            ("gemm fp8 %dx%dx%d (cmix value)" % (m, c, 4 * c), lambda s: self.gemm(s, synth.MAT_VALUE),
             4 * c * c + 4 * c, self.copies, fl(c, 4 * c)),
        ]


class Sweep:
    """The 13.3B decode step: 61 width-4096 layers of int4 g64 projections
    (fused R/K/V, O, cmix key, cmix value) and the fp16 65536x4096 head, all
    resident (7.06 GB), one graph per batch size; the activations are reused
    across layers (the step's data dependencies are not modelled)."""

    LAYERS, C, VOCAB = 61, 4096, 65536

    def __init__(self, gen, dev):
        c = self.C
        self.layers = []
        for _ in range(self.LAYERS):
            s = {}
            for mat, n, k in synth.layer_shapes(c):
                wf = torch.randn(n, k, generator=gen, device=dev, dtype=torch.float32) * (1.0 / k ** 0.5)
                s[mat] = rq.quantize(wf, rq.RQ_W4_SYM, 64)
                del wf
            self.layers.append(s)
        wf = torch.randn(self.VOCAB, c, generator=gen, device=dev, dtype=torch.float32) * (1.0 / c ** 0.5)
        self.head = rq.quantize(wf, rq.RQ_F16)
        del wf
        torch.cuda.empty_cache()
        self.weight_bytes = sum(q.nbytes() for s in self.layers for q in s.values()) + self.head.nbytes()
        self.x = {}
        self.y = {}

    def step(self, m):
        c = self.C
        if m not in self.x:
            self.x[m] = (f16_dev(synth.act_normal(m, c, 4), "cuda"), f16_dev(synth.act_normal(m, 4 * c, 4, salt=1), "cuda"))
            self.y[m] = {nm: torch.empty(m * n, dtype=torch.int16, device="cuda")
                         for nm, n in (("r", c), ("k", c), ("v", c), ("o", c), ("key", 4 * c), ("val", c),
                                       ("head", self.VOCAB))}
        x, x4 = self.x[m]
        y = self.y[m]
        for s in self.layers:
            rq.rq_fused_rkv(x, x, x, m, c, s[synth.MAT_R], s[synth.MAT_K], s[synth.MAT_V], y["r"], y["k"], y["v"], c)
            rq.rq_gemm_small_m(x, m, c, s[synth.MAT_O], y["o"], c)
            rq.rq_gemm_small_m(x, m, c, s[synth.MAT_KEY], y["key"], 4 * c)
            rq.rq_gemm_small_m(x4, m, 4 * c, s[synth.MAT_VALUE], y["val"], c)
        rq.rq_gemm_small_m(x, m, c, self.head, y["head"], self.VOCAB)

    def run(self, steps, warmup):
        out = {}
        for m in (1, 2, 4, 8, 16, 32):
            g = capture(lambda m=m: self.step(m))
            ms = time_graph(g, steps, warmup, launches=4 * self.LAYERS + 1)
            out[str(m)] = {"ms": round(ms, 4), "GB_s": round(self.weight_bytes / (ms * 1e-3) / 1e9, 1)}
            del g
        return out


class Ceiling:
    """The measured read ceiling: rq_stream_read (16-byte non-temporal loads
    over every compute unit) over a 4 GiB buffer, and over slices of it the
    size of one product's weights, launched back to back in a graph over
    distinct slices (as the products' classes rotate weight copies)."""

    BYTES = 4 << 30

    def __init__(self, dev):
        self.buf = torch.empty(self.BYTES, dtype=torch.uint8, device=dev)
        self.buf.fill_(1)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        g = capture(lambda: rq.rq_stream_read(self.buf, self.BYTES, self.sink))
        self.ms = time_graph(g, 20, launches=1)
        self.gbs = self.BYTES / (self.ms * 1e-3) / 1e9

    def per_launch_us(self, nbytes, launches=61):
        """Median per-launch time of a plain read of nbytes (16-byte multiple)."""
        nb = nbytes // 256 * 256
        slots = max(1, self.BYTES // nb)
        views = [self.buf[(i % slots) * nb:(i % slots) * nb + nb] for i in range(launches)]
        g = capture(lambda: [rq.rq_stream_read(v, nb, self.sink) for v in views])
        return time_graph(g, 5, launches=launches) * 1e3 / launches


def class_row(us, wbytes, ceiling, read_us=None):
    gbs = wbytes / us / 1e3
    out = {"us": round(us, 3), "weight_bytes": int(wbytes), "GB_s": round(gbs, 1),
           "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4), "ceiling_frac": round(gbs / ceiling.gbs, 4)}
    if read_us is not None:
        out["plain_read_us"] = round(read_us, 3)
        out["vs_plain_read"] = round(us / read_us, 3)
    return out


def sweep_classes(sw, ceiling, m=1):
    """Per-launch time of each launch class of the 13.3B step at M = m, each
    in a graph over the 61 layers' weights (the head alone: 537 MB, beyond the
    256 MB last-level cache), beside a plain read of the same bytes; and the
    sum over the step's 245 launches of those per-launch times."""
    c = sw.C
    x = f16_dev(synth.act_normal(m, c, 4), "cuda")
    x4 = f16_dev(synth.act_normal(m, 4 * c, 4, salt=1), "cuda")
    y = {nm: torch.empty(m * n, dtype=torch.int16, device="cuda")
         for nm, n in (("r", c), ("k", c), ("v", c), ("o", c), ("key", 4 * c), ("val", c), ("head", sw.VOCAB))}
    L = sw.layers
    kinds = [
        ("fused R/K/V 3x4096x4096", lambda s: rq.rq_fused_rkv(x, x, x, m, c, s[synth.MAT_R], s[synth.MAT_K],
                                                              s[synth.MAT_V], y["r"], y["k"], y["v"], c),
         sum(L[0][t].nbytes() for t in (synth.MAT_R, synth.MAT_K, synth.MAT_V))),
        ("O 4096x4096", lambda s: rq.rq_gemm_small_m(x, m, c, s[synth.MAT_O], y["o"], c), L[0][synth.MAT_O].nbytes()),
        ("cmix key 16384x4096", lambda s: rq.rq_gemm_small_m(x, m, c, s[synth.MAT_KEY], y["key"], 4 * c),
         L[0][synth.MAT_KEY].nbytes()),
        ("cmix value 4096x16384", lambda s: rq.rq_gemm_small_m(x4, m, 4 * c, s[synth.MAT_VALUE], y["val"], c),
         L[0][synth.MAT_VALUE].nbytes()),
    ]
    out = {}
    step_ms = 0.0
    for name, fn, wb in kinds:
        g = capture(lambda fn=fn: [fn(s) for s in L])
        us = time_graph(g, 5, launches=len(L)) * 1e3 / len(L)
        del g
        out[name] = class_row(us, wb, ceiling, ceiling.per_launch_us(wb))
        step_ms += len(L) * us * 1e-3
    g = capture(lambda: rq.rq_gemm_small_m(x, m, c, sw.head, y["head"], sw.VOCAB))
    us = time_graph(g, 5, launches=1) * 1e3
    del g
    out["head 65536x4096"] = class_row(us, sw.head.nbytes(), ceiling, ceiling.per_launch_us(sw.head.nbytes(), 8))
    step_ms += us * 1e-3
    return out, step_ms


def w8_rows(gen, dev, ceiling, copies=5):
    """The int8 tier (w8g64) of the 13.3B shapes at M = 1: each class over
    `copies` layers of distinct weights (1 GB), per-launch time beside a plain
    read of the same bytes."""
    c, m = 4096, 1
    layers = []
    for _ in range(copies):
        s = {}
        for mat, n, k in synth.layer_shapes(c):
            wf = torch.randn(n, k, generator=gen, device=dev, dtype=torch.float32) * (1.0 / k ** 0.5)
            s[mat] = rq.quantize(wf, rq.RQ_W8_SYM, 64)
            del wf
        layers.append(s)
    torch.cuda.empty_cache()
    x = f16_dev(synth.act_normal(m, c, 4), dev)
    x4 = f16_dev(synth.act_normal(m, 4 * c, 4, salt=1), dev)
    y = torch.empty(4 * c * 3, dtype=torch.int16, device=dev)
    yv = [y[i * c:(i + 1) * c] for i in range(3)]
    out = {}
    for name, fn, mats in (
            ("fused R/K/V 3x4096x4096", lambda s: rq.rq_fused_rkv(x, x, x, m, c, s[synth.MAT_R], s[synth.MAT_K],
                                                                  s[synth.MAT_V], yv[0], yv[1], yv[2], c),
             (synth.MAT_R, synth.MAT_K, synth.MAT_V)),
            ("O 4096x4096", lambda s: rq.rq_gemv_w8g64(x, s[synth.MAT_O], y), (synth.MAT_O,)),
            ("cmix key 16384x4096", lambda s: rq.rq_gemv_w8g64(x, s[synth.MAT_KEY], y), (synth.MAT_KEY,)),
            ("cmix value 4096x16384", lambda s: rq.rq_gemv_w8g64(x4, s[synth.MAT_VALUE], y), (synth.MAT_VALUE,))):
        g = capture(lambda fn=fn: [fn(s) for s in layers])
        us = time_graph(g, 20, launches=len(layers)) * 1e3 / len(layers)
        del g
        wb = sum(layers[0][t].nbytes() for t in mats)
        out[name] = class_row(us, wb, ceiling, ceiling.per_launch_us(wb, 20))
    del layers
    torch.cuda.empty_cache()
    return out


def _w4_gemm_rows(gen, dev, c, fmt, group, ms, label, graph_us):
    """rq_gemm_w4 on 6 copies of the width-c set: us per set and TFLOP/s."""
    out = {}
    wsets = []
    for _ in range(6):
        wset = {}
        for mat, n, k in synth.layer_shapes(c):
            wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
            wset[mat] = rq.quantize(wf, fmt, group)
            del wf
        wsets.append(wset)
    for m in ms:
        xa = f16_dev(synth.act_normal(m, c, 3), dev)
        xa4 = f16_dev(synth.act_normal(m, 4 * c, 3, salt=1), dev)
        yp = torch.empty(m * 4 * c, dtype=torch.int16, device=dev)

        def w4_pass(m=m, xa=xa, xa4=xa4, yp=yp):
            for wset in wsets:
                for mat in (synth.MAT_R, synth.MAT_K, synth.MAT_V, synth.MAT_O, synth.MAT_KEY):
                    rq.rq_gemm_w4(xa, m, c, wset[mat], yp, wset[mat].n)
                rq.rq_gemm_w4(xa4, m, 4 * c, wset[synth.MAT_VALUE], yp, c)
        us = graph_us(w4_pass, len(wsets))
        flops = sum(2.0 * m * n * k for _, n, k in synth.layer_shapes(c))
        out["%s gemm %d set M=%d" % (label, c, m)] = {
            "us_per_set": round(us, 2), "TFLOPS": round(flops / us / 1e6, 1),
            "frac_of_fp16_peak": round(flops / us / 1e6 / F16_PEAK_TFLOPS, 4)}
    del wsets
    return out


class PresetSweep:
    """Decode steps of the 2.9B shape (32 layers of width 2560, head
    65536x2560) with every tensor in the format its rwkv-quant preset assigns
    (gemm_rwkv_amd.presets): REDUCTION, COMPRESSION, and COMPRESSION with the
    first block's output projection in bf16.  Weights are quantized on the GPU
    from seeded normal fp32 matrices; one graph per (preset, M), activations
    reused across layers as in Sweep."""

    LAYERS, C, VOCAB = 32, 2560, 65536
    NAMES = ("r", "k", "v", "o", "cmix_key", "cmix_value")

    def __init__(self, gen, dev):
        c = self.C
        self.layers = {}
        self.heads = {}
        self.bf16_o0 = None
        for name in presets.PRESETS:
            ls = []
            for li in range(self.LAYERS):
                s = {}
                for (mat, n, k), tn in zip(synth.layer_shapes(c), self.NAMES):
                    wf = torch.randn(n, k, generator=gen, device=dev, dtype=torch.float32) * (1.0 / k ** 0.5)
                    fmt, group = presets.scheme(name, tn, li)
                    s[tn] = rq.quantize(wf, fmt, group)
                    if name == "COMPRESSION" and tn == "o" and li == 0:
                        self.bf16_o0 = rq.quantize(wf, *presets.BF16_FIRST_O)
                    del wf
                ls.append(s)
            self.layers[name] = ls
            wf = torch.randn(self.VOCAB, c, generator=gen, device=dev, dtype=torch.float32) * (1.0 / c ** 0.5)
            self.heads[name] = rq.quantize(wf, *presets.scheme(name, "head", 0))
            del wf
        torch.cuda.empty_cache()
        self.x = {}
        self.y = {}

    def variants(self):
        return (("REDUCTION", "REDUCTION", False), ("COMPRESSION", "COMPRESSION", False),
                ("COMPRESSION+bf16_o0", "COMPRESSION", True))

    def weight_bytes(self, name, bf16_o0):
        b = sum(q.nbytes() for s in self.layers[name] for q in s.values()) + self.heads[name].nbytes()
        if bf16_o0:
            b += self.bf16_o0.nbytes() - self.layers[name][0]["o"].nbytes()
        return b

    def step(self, name, bf16_o0, m):
        c = self.C
        if m not in self.x:
            self.x[m] = (f16_dev(synth.act_massive(m, c, cfg=2, salt=1), "cuda"),
                         f16_dev(synth.act_massive(m, 4 * c, cfg=2, salt=2), "cuda"))
            self.y[m] = {nm: torch.empty(m * n, dtype=torch.int16, device="cuda")
                         for nm, n in (("r", c), ("k", c), ("v", c), ("o", c), ("key", 4 * c), ("val", c),
                                       ("head", self.VOCAB))}
        x, x4 = self.x[m]
        y = self.y[m]
        for li, s in enumerate(self.layers[name]):
            o = self.bf16_o0 if (bf16_o0 and li == 0) else s["o"]
            rq.rq_fused_rkv(x, x, x, m, c, s["r"], s["k"], s["v"], y["r"], y["k"], y["v"], c)
            rq.rq_gemm_small_m(x, m, c, o, y["o"], c)
            rq.rq_gemm_small_m(x, m, c, s["cmix_key"], y["key"], 4 * c)
            rq.rq_gemm_small_m(x4, m, 4 * c, s["cmix_value"], y["val"], c)
        rq.rq_gemm_small_m(x, m, c, self.heads[name], y["head"], self.VOCAB)

    def run(self, steps, warmup):
        out = {}
        for label, name, b16 in self.variants():
            wb = self.weight_bytes(name, b16)
            per_m = {}
            for m in (1, 4, 16):
                g = capture(lambda m=m: self.step(name, b16, m))
                ms = time_graph(g, steps, warmup, launches=129)
                per_m[str(m)] = {"ms": round(ms, 4), "GB_s": round(wb / (ms * 1e-3) / 1e9, 1)}
                del g
            out[label] = {"weight_bytes": wb, "per_m": per_m}
        return out


def measure_rows(gen, dev, reps=20):
    """One measurement per row of the path that the step does not time: the
    quantizers, the SB256 products (width 2560, M = 1, 4, 16), the int8 GEMM
    (width 4096 prefill set, M = 256), the width-768 fused R/K/V call and the
    fp16 head at M = 1.  Each is the mean of `reps` back-to-back launches in
    a graph over distinct weight copies where the weights are large."""
    out = {}

    def graph_us(fn, n):
        g = capture(fn)
        return time_graph(g, reps, launches=n) * 1e3 / n

    # quantizers: fp32 bytes read per second
    for name, fmt, group, (n, k) in (("rtn w4g64 8192x2048", rq.RQ_W4_SYM, 64, (8192, 2048)),
                                     ("rtn sb256 10240x2560", rq.RQ_W4_ASYM_SB256, 32, (10240, 2560)),
                                     ("rtn fp8 per-channel 16384x4096", rq.RQ_FP8_E4M3_CH, 0, (16384, 4096))):
        wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
        q = rq.QWeight.empty(fmt, group, n, k, device=dev)
        rq.rq_quantize_rtn(wf, q)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            rq.rq_quantize_rtn(wf, q)  # synchronizes (reads back its status word)
        us = (time.perf_counter() - t0) * 1e6 / 5
        out[name] = {"us": round(us, 2), "GB_s_fp32_in": round(n * k * 4 / us / 1e3, 1)}
        del wf, q
    # activation-weighted search (16 candidates per group), importance from a
    # massive-channel batch
    for name, fmt, group, (n, k) in (("aw w4g64 8192x2048", rq.RQ_W4_SYM, 64, (8192, 2048)),
                                     ("aw sb256 10240x2560", rq.RQ_W4_ASYM_SB256, 32, (10240, 2560))):
        wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
        xc = torch.from_numpy(synth.act_massive(256, k, cfg=2, salt=1)).to(dev).float()
        a = (xc * xc).mean(0).contiguous()
        q = rq.QWeight.empty(fmt, group, n, k, device=dev)
        rq.rq_quantize_aw(wf, a, q)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            rq.rq_quantize_aw(wf, a, q)
        us = (time.perf_counter() - t0) * 1e6 / 5
        out[name] = {"us": round(us, 2), "GB_s_fp32_in": round(n * k * 4 / us / 1e3, 1)}
        del wf, xc, a, q
    # SB256 products, width 2560, 32 copies of the set
    c = 2560
    sets = []
    for _ in range(32):
        sset = {}
        for mat, n, k in ((synth.MAT_O, c, c), (synth.MAT_KEY, 4 * c, c), (synth.MAT_VALUE, c, 4 * c)):
            wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
            sset[mat] = rq.quantize(wf, rq.RQ_W4_ASYM_SB256, 32)
            del wf
        sets.append(sset)
    for m in (1, 4, 16):
        x = f16_dev(synth.act_massive(m, c), dev)
        x4 = f16_dev(synth.act_massive(m, 4 * c), dev)
        y = torch.empty(m * 4 * c, dtype=torch.int16, device=dev)

        def sb_pass(m=m, x=x, x4=x4, y=y):
            for sset in sets:
                rq.rq_gemm_small_m(x, m, c, sset[synth.MAT_O], y, c)
                rq.rq_gemm_small_m(x, m, c, sset[synth.MAT_KEY], y, 4 * c)
                rq.rq_gemm_small_m(x4, m, 4 * c, sset[synth.MAT_VALUE], y, c)
        us = graph_us(sb_pass, len(sets))
        wb = sum(q.nbytes() for q in sets[0].values())
        out["sb256 2560 set M=%d" % m] = {"us_per_set": round(us, 2), "GB_s": round(wb / us / 1e3, 1),
                                           "hbm_peak_frac": round(wb / us / 1e3 / HBM_PEAK_GBS, 4)}
    del sets
    # fp8 prefill set (activation quantization included, as in the step) at
    # the other prefill chunk sizes, M = 64 and 1024
    for m in (64, 1024):
        pm = Prefill(4096, m, gen, dev)
        us = graph_us(pm.passes, pm.copies)
        out["fp8 gemm 4096 set M=%d" % m] = {"us_per_set": round(us, 2),
                                             "TFLOPS": round(pm.flops / us / 1e6, 1),
                                             "frac_of_peak": round(pm.flops / us / 1e6 / FP8_PEAK_TFLOPS, 4)}
        del pm
        torch.cuda.empty_cache()
    # int8 GEMM, width-4096 prefill set at M = 256, 6 copies
    c, m = 4096, 256
    isets = []
    for _ in range(6):
        iset = {}
        for mat, n, k in synth.layer_shapes(c):
            wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
            iset[mat] = rq.quantize(wf, rq.RQ_I8_CH)
            del wf
        isets.append(iset)
    xa = f16_dev(synth.act_normal(m, c, 3), dev)
    xa4 = f16_dev(synth.act_normal(m, 4 * c, 3, salt=1), dev)
    xq = torch.empty(m * c, dtype=torch.uint8, device=dev)
    xq4 = torch.empty(m * 4 * c, dtype=torch.uint8, device=dev)
    sx = torch.empty(m, dtype=torch.float32, device=dev)
    sx4 = torch.empty(m, dtype=torch.float32, device=dev)
    yp = torch.empty(m * 4 * c, dtype=torch.int16, device=dev)
    rq.rq_quantize_act(xa, m, c, c, rq.RQ_I8_CH, xq, sx)
    rq.rq_quantize_act(xa4, m, 4 * c, 4 * c, rq.RQ_I8_CH, xq4, sx4)

    def i8_pass():
        for iset in isets:
            for mat in (synth.MAT_R, synth.MAT_K, synth.MAT_V, synth.MAT_O, synth.MAT_KEY):
                rq.rq_gemm_int8(xq, sx, m, iset[mat], yp, iset[mat].n)
            rq.rq_gemm_int8(xq4, sx4, m, iset[synth.MAT_VALUE], yp, c)
    us = graph_us(i8_pass, len(isets))
    flops = sum(2.0 * m * n * k for _, n, k in synth.layer_shapes(c))
    out["int8 gemm 4096 set M=256"] = {"us_per_set": round(us, 2), "TOPS": round(flops / us / 1e6, 1),
                                       "frac_of_peak": round(flops / us / 1e6 / FP8_PEAK_TFLOPS, 4)}
    del isets
    # int4 prefill GEMM (rq_gemm_w4), width-4096 set, 6 copies, fp16
    # activations: symmetric g64 at M = 64, 256, 1024 (640 MB), superblocks
    # at M = 256 (340 MB)
    for fmt, group, ms, label in ((rq.RQ_W4_SYM, 64, (64, 256, 1024), "int4 g64"),
                                  (rq.RQ_W4_ASYM_SB256, 32, (256,), "int4 sb256")):
        out.update(_w4_gemm_rows(gen, dev, c, fmt, group, ms, label, graph_us))
    # width-768 fused R/K/V, w8g64, M = 1: 200 calls on distinct weight copies
    # (365 MB) per graph, so the figure is the per-call device time
    ws, x = synth.fused_rkv_768()
    q0 = [rq.quantize(torch.from_numpy(w).to(dev), rq.RQ_W8_SYM, 64) for w in ws]
    copies = []
    for _ in range(200):
        cq = []
        for q in q0:
            c_ = rq.QWeight.empty(q.format, q.group, q.n, q.k, device=dev)
            c_.codes.copy_(q.codes)
            c_.scales.copy_(q.scales)
            cq.append(c_)
        copies.append(cq)
    xd = f16_dev(x, dev)
    ys = [torch.empty(768, dtype=torch.int16, device=dev) for _ in range(3)]
    us = graph_us(lambda: [rq.rq_fused_rkv(xd, xd, xd, 1, 768, *cq, *ys, 768) for cq in copies], len(copies))
    wb = sum(q.nbytes() for q in q0)
    out["fused rkv 768 w8g64 M=1"] = {"us": round(us, 2), "GB_s": round(wb / us / 1e3, 1)}
    del copies
    # fp16 head 65536 x 4096 at M = 1, two copies (1.07 GB) per graph
    heads = []
    for _ in range(2):
        wf = torch.randn(65536, 4096, generator=gen, device=dev) * (1.0 / 64.0)
        heads.append(rq.quantize(wf, rq.RQ_F16))
        del wf
    xh = f16_dev(synth.act_normal(1, 4096, 4), dev)
    yh = torch.empty(65536, dtype=torch.int16, device=dev)
    us = graph_us(lambda: [rq.rq_gemv_f16(xh, h, yh) for h in heads], len(heads))
    hb = heads[0].nbytes()
    out["head f16 65536x4096 M=1"] = {"us": round(us, 2), "GB_s": round(hb / us / 1e3, 1),
                                      "hbm_peak_frac": round(hb / us / 1e3 / HBM_PEAK_GBS, 4)}
    return out


def class_graph(launch, sets):
    """One graph: the kernel class launched once per rotated weight copy."""
    return capture(lambda: [launch(s) for s in sets])


def measure_classes(dec, pre, reps):
    """Average launch duration (ms) of every kernel class, back to back in a graph."""
    rows = []
    for m in MS:
        for name, fn, wbytes, per_step in dec.classes(m):
            g = class_graph(fn, dec.sets)
            ms = time_graph(g, reps, launches=len(dec.sets)) / len(dec.sets)
            rows.append({"name": name, "ms": ms, "weight_bytes": wbytes, "per_step": per_step, "flops": 0.0,
                         "m": m, "graph": g, "launches": len(dec.sets)})
    for name, fn, wbytes, per_step, flops in pre.classes():
        g = class_graph(fn, pre.sets)
        ms = time_graph(g, reps, launches=len(pre.sets)) / len(pre.sets)
        rows.append({"name": name, "ms": ms, "weight_bytes": wbytes, "per_step": per_step, "flops": flops,
                     "m": pre.m, "graph": g, "launches": len(pre.sets)})
    return rows


FP8_RIDGE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per HBM byte


def roofline(row, traffic=None):
    """Roofline of one kernel class from its average launch duration: the
    algorithmic bytes (weights, scales, x, y) per launch against 8 TB/s, or,
    for a product above the fp8 ridge, its flops against the fp8 MFMA peak."""
    sec = row["ms"] * 1e-3
    out = {"kernel": row["name"], "launch_us": round(row["ms"] * 1e3, 3),
           "alg_bytes_per_launch": int(row["alg_bytes"])}
    if row["flops"] > 0:
        out["tflops"] = round(row["flops"] / sec / 1e12, 2)
    if row["flops"] > 0 and row["flops"] / row["alg_bytes"] >= FP8_RIDGE:
        a = row["flops"] / sec / 1e12
        out.update({"bound": "mfma", "achieved": round(a, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a / FP8_PEAK_TFLOPS, 4)})
    else:
        a = row["alg_bytes"] / sec / 1e9
        out.update({"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(a / HBM_PEAK_GBS, 4)})
    out["traffic"] = traffic
    return out


def alg_bytes(row, c1, c3, m3):
    """Algorithmic HBM bytes of one launch: weights (+ scales), x and y."""
    name, m = row["name"], row["m"]
    if "act quant" in name:
        k = 4 * c3 if "x%d" % (4 * c3) in name else c3
        return m3 * k * 2 + m3 * k + 4 * m3
    if row["flops"] > 0:
        n_k = row["flops"] / (2.0 * m3)
        k = 4 * c3 if "value" in name else c3
        n = n_k / k
        return row["weight_bytes"] + m3 * k + 4 * m3 + m3 * n * 2
    if "fused" in name:
        return row["weight_bytes"] + 3 * m * c1 * 2 + 3 * m * c1 * 2
    if "cmix key" in name:
        return row["weight_bytes"] + m * c1 * 2 + m * 4 * c1 * 2
    if "cmix value" in name:
        return row["weight_bytes"] + m * 4 * c1 * 2 + m * c1 * 2
    return row["weight_bytes"] + 2 * m * c1 * 2


def _wide(name):
    """A decode class of the width-4096 layer (the 13.3B shapes)."""
    return "gemv" in name and ("4096x" in name or "x4096" in name)


def kernel_only(dec, pre, name, steps, dev, gen=None):
    """Counter run: one calibration copy of CALIB_BYTES, then the class graph
    replayed `steps` times; every dispatch after the last copy belongs to it.
    Classes of the width-4096 layer (e.g. "gemv w4g64 cmix key 16384x4096
    M=1") run over rotated copies of that layer instead."""
    if name and _wide(name):
        dec = Decode(4096, gen, dev)
    classes = [(n, fn, dec.sets) for m in MS for n, fn, _, _ in dec.classes(m)]
    classes += [(n, fn, pre.sets) for n, fn, _, _, _ in pre.classes()]
    if not name:
        rows = measure_classes(dec, pre, 1)
        name = max(rows, key=lambda r: r["ms"] * r["per_step"])["name"]
    match = [c for c in classes if c[0] == name]
    if not match:
        sys.exit("no kernel class named %r" % name)
    _, fn, sets = match[0]
    g = class_graph(fn, sets)
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    print("kernel-only: %s, %d launches per replay, %d replays, after a %d-byte calibration copy"
          % (name, len(sets), steps, CALIB_BYTES), file=sys.stderr)


def _counter_rows(path):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def traffic_from(fetch_csv, write_csv):
    """HBM bytes per launch of a --kernel-only class: every dispatch after the
    last calibration copy, scaled by what the counters read for that copy."""
    res = {}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _counter_rows(path)
        ids = sorted(rows)
        copies = [d for d in ids if "copyBuffer" in rows[d][0] or "copy" in rows[d][0].lower()]
        if not copies:
            sys.exit("%s: no calibration copy dispatch found" % path)
        c = copies[-1]
        calib = rows[c][1] * 1024.0  # the counters read KiB
        after = [d for d in ids if d > c]
        total = sum(rows[d][1] for d in after) * 1024.0
        res[label] = (calib, total, len(after), sorted({rows[d][0].split("(")[0] for d in after}))
    return res


def trace_summary(path, after_copy=False):
    """Library kernels of a rocprofv3 kernel trace grouped by name and launch
    shape (workgroups x threads): dispatches, mean and median duration.  With
    after_copy, only the dispatches after the last device copy (the
    calibration copy of a --kernel-only run)."""
    import csv
    groups = {}
    with open(path) as f:
        rows = list(csv.DictReader(f))
    t0 = 0
    if after_copy:
        ends = [int(r["End_Timestamp"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        t0 = max(ends) if ends else 0
    for r in rows:
        if True:
            name = r["Kernel_Name"]
            if "rq::" not in name or int(r["Start_Timestamp"]) < t0:
                continue
            short = name.split("(")[0].replace("void ", "")
            wg = int(r["Workgroup_Size_X"])
            key = (short, int(r["Grid_Size_X"]) // wg * int(r.get("Grid_Size_Y", 1) or 1), wg)
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("%-44s %9s %7s %9s %10s %10s" % ("kernel", "wgs", "threads", "dispatches", "mean_us", "median_us"))
    for (short, wgs, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        print("%-44s %9d %7d %9d %10.2f %10.2f" % (short[:44], wgs, wg, len(v), sum(v) / len(v) / 1e3,
                                                  v[len(v) // 2] / 1e3))


def copies_for(name):
    """Weight copies in rotation for a kernel class (without a GPU)."""
    if "fp8" in name:
        per_set = sum(n * k + 4 * n for _, n, k in synth.layer_shapes(C3))
    else:
        c = 4096 if _wide(name) else C1
        per_set = sum(sum(rq.rq_qweight_bytes(rq.RQ_W4_SYM, 64, n, k)[:2]) for _, n, k in synth.layer_shapes(c))
    return -(-ROTATE_BYTES // per_set)


def print_traffic(csvs, name, steps):
    """The lines of profiles/traffic.txt for class `name` (a --kernel-only run
    with `steps` replays), from the FETCH_SIZE and WRITE_SIZE counter CSVs."""
    if not name:
        sys.exit("--traffic-from needs the class name in --kernel-only")
    res = traffic_from(*csvs)
    launches = steps * copies_for(name)
    per = {}
    for label in ("fetch", "write"):
        calib, total, ndisp, kernels = res[label]
        per[label] = total / calib * CALIB_BYTES / launches
    print("class: %s" % name)
    print("bytes_per_launch: %.0f" % (per["fetch"] + per["write"]))
    print("fetch_bytes_per_launch: %.0f" % per["fetch"])
    print("write_bytes_per_launch: %.0f" % per["write"])
    for label, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        calib, total, ndisp, kernels = res[label]
        print("%s_calibration: %s read %.0f KiB for the %d-byte copy (factor %.4f); %d dispatches after it: %s"
              % (label, ctr, calib / 1024, CALIB_BYTES, CALIB_BYTES / calib, ndisp, ", ".join(kernels)))
    print("launches: %d" % launches)
    print("sources_sha256: %s" % sources_hash(name))


def stored_traffic(name):
    """Counter-derived bytes per launch for kernel class `name` from
    profiles/traffic.txt, or None when absent, for another class, or taken
    from kernel sources that have changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("class") != name or fields.get("sources_sha256") != sources_hash(name):
        return None
    try:
        return float(fields["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def sources_hash(name):
    """SHA-256 over the sources the kernel class `name` is built from: its own
    kernel file plus the shared headers and the C-ABI layer that plans and
    launches it.  A change to an unrelated kernel file leaves it unchanged."""
    import hashlib
    if "gemm" in name:
        own = "gemm_mfma.hip"
    elif "quant" in name:
        own = "quant.hip"
    else:
        own = "gemv.hip"
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_rwkv_amd", "csrc")
    for fn in sorted([own, "api.hip", "device_common.h", "kernels.h"]):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(c, budget_s):
    """Whole width-c layers through the oracle at M = 1, 8, 32 until budget_s
    is spent: (packed weight bytes of the passes, seconds, layers)."""
    from oracle import quant, ref
    xs = {m: synth.act_channel_1202(m, c) for m in MS}
    x4 = {m: synth.act_normal(m, 4 * c, 1) for m in MS}
    t0 = time.perf_counter()
    nbytes = 0
    layers = 0
    while True:
        for mat, n, k in synth.layer_shapes(c):
            w = synth.weight(1, layers, mat, n, k)
            parts = quant.quantize_sym(w, 4, 64)
            nbytes += len(MS) * (parts["codes"].nbytes + parts["scales"].nbytes)
            for m in MS:
                x = xs[m] if k == c else x4[m]
                ref.weight_only_ref(x, quant.W4_SYM, parts, 64)
        layers += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return nbytes, time.perf_counter() - t0, layers


def cpu_baseline(c, budget_s=12.0):
    """The oracle (RTN quantize, dequantize, fp64 product) on host cores over a
    bounded sample of the decode step: whole width-c layers at M = 1, 8, 32,
    once with the BLAS threads numpy has and once on one thread."""
    threads = os.cpu_count()
    limits = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        limits = threadpool_limits
    except Exception:  # noqa: BLE001
        pass
    nb, dt, layers = _oracle_pass(c, budget_s)
    out = {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": "%d layer(s) of the width-%d int4 g64 set (6 matrices) through the oracle's RTN "
                     "quantizer, dequantization and fp64 product at M=1,8,32: %.1f s; value = packed "
                     "weight bytes of the decode passes / time" % (layers, c, dt),
           "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}
    if limits is not None:
        with limits(limits=1):
            nb1, dt1, layers1 = _oracle_pass(c, budget_s)
        out["single_thread"] = {"value": round(nb1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "sample": "%d layer(s), %.1f s, BLAS limited to one thread" % (layers1, dt1)}
    return out


def vendor_gemm(gen, dev, ms=(64, 256, 1024), reps=20):
    """Context, not the product: the library's fp8 and int8 GEMMs beside the
    vendor library's (hipBLASLt through torch._scaled_mm with per-tensor
    scales and fp16 output, and torch._int_mm) at the 7.2B-width prefill
    shapes.  Each side runs back to back over rotated weight copies (over
    1 GiB) in one captured graph per shape; activations are quantized
    beforehand.  us per product, median over at least 200 dispatches."""
    shapes = [("R/K/V/O", C3, C3), ("cmix key", 4 * C3, C3), ("cmix value", C3, 4 * C3)]
    out = {}
    for name, n, k in shapes:
        copies = max(4, -(-ROTATE_BYTES // (n * k)))
        ours8 = [rq.quantize(torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5), rq.RQ_FP8_E4M3_CH)
                 for _ in range(copies)]
        ours_i = [rq.quantize(torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5), rq.RQ_I8_CH)
                  for _ in range(copies)]
        # the vendor side multiplies the same code bytes, viewed as torch fp8 / int8 tensors [n][k]
        v8 = [w.codes.view(torch.float8_e4m3fn).view(n, k) for w in ours8]
        vi = [w.codes.view(torch.int8).view(n, k) for w in ours_i]
        one = torch.ones((), device=dev, dtype=torch.float32)
        for m in ms:
            xa = f16_dev(synth.act_normal(m, k, 3), dev)
            xq = torch.empty(m * k, dtype=torch.uint8, device=dev)
            xqi = torch.empty(m * k, dtype=torch.uint8, device=dev)
            sx = torch.empty(m, dtype=torch.float32, device=dev)
            sxi = torch.empty(m, dtype=torch.float32, device=dev)
            rq.rq_quantize_act(xa, m, k, k, rq.RQ_FP8_E4M3_CH, xq, sx)
            rq.rq_quantize_act(xa, m, k, k, rq.RQ_I8_CH, xqi, sxi)
            y = torch.empty(m * n, dtype=torch.int16, device=dev)
            x8 = xq.view(torch.float8_e4m3fn).view(m, k)
            x8i = xqi.view(torch.int8).view(m, k)
            fl = 2.0 * m * n * k
            row = {}
            legs = [("fp8 library", lambda: [rq.rq_gemm_fp8(xq, sx, m, w, y, n) for w in ours8]),
                    ("fp8 hipBLASLt", lambda: [torch._scaled_mm(x8, w.t(), scale_a=one, scale_b=one,
                                                                out_dtype=torch.float16) for w in v8]),
                    ("int8 library", lambda: [rq.rq_gemm_int8(xqi, sxi, m, w, y, n) for w in ours_i]),
                    ("int8 hipBLASLt", lambda: [torch._int_mm(x8i, w.t()) for w in vi])]
            for leg, fn in legs:
                try:
                    us = time_graph(capture(fn), reps, launches=copies) * 1e3 / copies
                    row[leg] = {"us": round(us, 2), "TFLOP_s": round(fl / us / 1e6, 1)}
                except Exception as e:  # a vendor path this torch build does not offer
                    row[leg] = {"error": "%s: %s" % (type(e).__name__, str(e)[:160])}
                torch.cuda.synchronize()
            out["%s %dx%d M=%d" % (name, n, k, m)] = row
            print("%-28s %s" % ("%s %dx%d M=%d" % (name, n, k, m), row), file=sys.stderr, flush=True)
        del ours8, ours_i, v8, vi
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phases", action="store_true", help="per-class timings to stderr")
    ap.add_argument("--kernel-only", nargs="?", const="", default=None, metavar="CLASS",
                    help="for counter runs: a calibration copy, then only the named kernel class "
                         "(default: the dominant one) replayed --steps times")
    ap.add_argument("--class-reps", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true", help="skip the 13.3B decode-step sweep")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    ap.add_argument("--no-presets", action="store_true", help="skip the 2.9B preset decode sweeps")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="per kernel and launch shape: dispatches and mean duration, from a "
                         "rocprofv3 --kernel-trace CSV")
    ap.add_argument("--prefill-m", type=int, default=M3,
                    help="with --kernel-only: the prefill classes at this M (default 256)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only the fp8/int8 GEMMs beside the vendor library's at the prefill shapes "
                         "(context), one JSON line")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of a --kernel-only run into HBM "
                         "bytes per launch (printed as the lines of a profiles/ summary)")
    args = ap.parse_args()
    if args.traffic_from:
        print_traffic(args.traffic_from, args.kernel_only, args.steps)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, after_copy=args.kernel_only is not None)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    if args.vendor_gemm:
        print(json.dumps({"vendor_gemm": vendor_gemm(gen, dev)}))
        return

    dec = Decode(C1, gen, dev)
    pre = Prefill(C3, args.prefill_m if args.kernel_only is not None else M3, gen, dev)
    if args.kernel_only is not None:
        print("weights ready", file=sys.stderr, flush=True)

    if args.kernel_only is not None:
        kernel_only(dec, pre, args.kernel_only, args.steps, dev, gen)
        return

    graphs = [capture(lambda m=m: dec.passes(m)) for m in MS] + [capture(pre.passes)]
    for _ in range(args.warmup):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
    per = np.zeros(len(graphs))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev[0].record()
        for i, g in enumerate(graphs):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per += [ev[i].elapsed_time(ev[i + 1]) for i in range(len(graphs))]
    wall = (time.perf_counter() - t0) * 1e3 / args.steps
    per /= args.steps
    dec_ms = float(per[:len(MS)].sum())
    value = len(MS) * dec.copies * dec.set_bytes / (dec_ms * 1e-3) / 1e9
    fp8_tflops = pre.copies * pre.flops / (per[-1] * 1e-3) / 1e12

    rows = measure_classes(dec, pre, args.class_reps)
    for r in rows:
        r["alg_bytes"] = alg_bytes(r, C1, C3, M3)
    dom = max(rows, key=lambda r: r["ms"] * r["per_step"])
    traffic = stored_traffic(dom["name"])
    ceiling = Ceiling(dev)
    if args.phases:
        for name, t in zip(["decode M=%d" % m for m in MS] + ["prefill fp8 M=%d" % M3], per):
            print("%-22s %8.3f ms" % (name, t), file=sys.stderr)
        for r in rows:
            rl = roofline(r)
            print("%-46s %8.2f us  x%-4d %7.1f %s (%.1f%%)" % (r["name"], r["ms"] * 1e3, r["per_step"],
                  rl["achieved"], rl["unit"], 100 * rl["frac"]), file=sys.stderr)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic: weights N(0,1/K) quantized on the GPU; x N(0,1) fp16, channel 1202 x50",
        "config": {"workload": "rwkv7 1.5B-width (C=2048) int4 sym g64 layer set (fused R/K/V, O, cmix "
                               "key, cmix value) decoded at M=1,8,32, then the 7.2B-width (C=4096) fp8 "
                               "per-channel prefill set at M=256",
                   "decode_copies": dec.copies, "decode_weight_bytes_per_set": dec.set_bytes,
                   "prefill_copies": pre.copies, "prefill_weight_bytes_per_set": pre.set_bytes,
                   "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
                   "decode_ms": {str(m): round(float(t), 4) for m, t in zip(MS, per)}},
        "fp8_gemm_m256": {"tflops": round(fp8_tflops, 1), "frac_of_peak": round(fp8_tflops / FP8_PEAK_TFLOPS, 4),
                          "pass_ms": round(float(per[-1]), 4)},
        "roofline": roofline(dom, traffic),
        "hbm_ceiling": {"GB_s": round(ceiling.gbs, 1), "bytes": Ceiling.BYTES, "ms": round(ceiling.ms, 4),
                        "peak_frac": round(ceiling.gbs / HBM_PEAK_GBS, 4),
                        "kernel": "rq_stream_read: 16-byte non-temporal loads, 8 per thread per step, "
                                  "grid-stride over all compute units"},
    }
    out["config"]["ceiling_frac"] = round(value / ceiling.gbs, 4)
    if out["roofline"]["unit"] == "GB/s":
        out["roofline"]["ceiling_frac"] = round(out["roofline"]["achieved"] / ceiling.gbs, 4)
    if not args.no_sweep:
        del graphs, rows
        torch.cuda.empty_cache()
        sw = Sweep(gen, dev)
        res = sw.run(max(3, args.steps // 2), 2)
        cls, sum_ms = sweep_classes(sw, ceiling)
        out["sweep_13b"] = {"workload": "61 x (fused R/K/V, O, cmix key, cmix value) int4 g64 at width 4096 "
                                        "+ fp16 head 65536x4096, one graph of 245 launches per M",
                            "weight_bytes": sw.weight_bytes, "per_m": res,
                            "m1_hbm_peak_frac": round(res["1"]["GB_s"] / HBM_PEAK_GBS, 4),
                            "m1_ceiling_frac": round(res["1"]["GB_s"] / ceiling.gbs, 4),
                            "m1_classes": cls,
                            "m1_sum_of_class_launches_ms": round(sum_ms, 4)}
        if args.phases:
            for name, r in cls.items():
                print("sweep M=1 %-26s %s" % (name, r), file=sys.stderr)
        if args.phases:
            for m, r in res.items():
                print("sweep 13.3B M=%-2s %8.3f ms  %7.1f GB/s" % (m, r["ms"], r["GB_s"]), file=sys.stderr)
        del sw
    if not args.no_presets:
        torch.cuda.empty_cache()
        ps = PresetSweep(gen, dev)
        res = ps.run(max(3, args.steps // 2), 2)
        out["presets_2p9b"] = {"workload": "32 x (fused R/K/V, O, cmix key, cmix value) at width 2560 + head "
                                           "65536x2560, each tensor in its rwkv-quant preset format, one graph "
                                           "of 129 launches per M", "variants": res}
        if args.phases:
            for label, r in res.items():
                for m, v in r["per_m"].items():
                    print("preset %-20s M=%-2s %8.3f ms  %7.1f GB/s" % (label, m, v["ms"], v["GB_s"]), file=sys.stderr)
        del ps
    if not args.no_rows:
        torch.cuda.empty_cache()
        out["rows"] = measure_rows(gen, dev)
        out["rows"]["w8g64 4096 layer M=1"] = w8_rows(gen, dev, ceiling)
        if args.phases:
            for name, r in out["rows"].items():
                print("%-34s %s" % (name, r), file=sys.stderr)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(C1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
