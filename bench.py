"""Benchmark of the quantized-weight decode and prefill products on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one decode pass of the RWKV-7 1.5B projection stack (24 layers x
{fused R/K/V, O, cmix key, cmix value}, symmetric int4 group 64, fp16
activations with the massive channel 1202) at each batch M in {1, 8, 32},
followed by one prefill pass of the 7.2B projection set (R, K, V, O, cmix key,
cmix value; per-token fp8 activations x per-channel fp8 weights) at M = 256.
Every pass is a captured HIP graph; inputs are resident in HBM before timing.

The JSON line's value is the int4 weight stream: packed weight bytes of the
decode passes / their wall time (GB/s, % of 8 TB/s).  The fp8 prefill GEMM
rate is reported beside it.  Synthetic weights: N(0, 1/K) drawn on the GPU
from a seeded generator, quantized with rq_quantize_rtn.
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
from gemm_rwkv_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
METRIC = "weight-stream GB/s (% HBM peak) W4g64 GEMV M=1..32; TFLOPS fp8 GEMM M=256"


def f16_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).view(np.int16)).to(dev)


class Layer:
    """The six quantized projections of one RWKV-7 layer (W[N][K])."""

    def __init__(self, c, fmt, group, gen, dev):
        self.w = {}
        for mat, n, k in synth.layer_shapes(c):
            wf = torch.randn(n, k, generator=gen, device=dev, dtype=torch.float32) * (1.0 / k ** 0.5)
            self.w[mat] = rq.quantize(wf, fmt, group)
            del wf

    def weight_bytes(self):
        return sum(q.nbytes() for q in self.w.values())


def decode_pass(layers, xc, x4c, y, m, c):
    """Launch one layer stack: fused R/K/V, O, cmix key, cmix value."""
    ldx = c
    for L in layers:
        w = L.w
        rq.rq_fused_rkv(xc, xc, xc, m, ldx, w[synth.MAT_R], w[synth.MAT_K], w[synth.MAT_V],
                        y["r"], y["k"], y["v"], c)
        rq.rq_gemm_small_m(xc, m, ldx, w[synth.MAT_O], y["o"], c)
        rq.rq_gemm_small_m(xc, m, ldx, w[synth.MAT_KEY], y["key"], 4 * c)
        rq.rq_gemm_small_m(x4c, m, 4 * c, w[synth.MAT_VALUE], y["val"], c)


def capture(fn):
    fn()  # eager run first: loads code objects outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed(graphs, steps, warmup):
    """Replay each graph per step; return per-graph mean ms (events) and wall ms/step."""
    for _ in range(warmup):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        for i, g in enumerate(graphs):
            g.replay()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]) for i in range(len(graphs))]
    return per, wall


def cpu_baseline(c, budget_s=20.0):
    """The oracle (dequantize + fp64 product) on host cores over a bounded
    sample of the decode pass: whole layers of the width-c stack at M = 1, 8, 32."""
    from oracle import quant, ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    xs = {m: synth.act_channel_1202(m, c) for m in (1, 8, 32)}
    x4 = {m: synth.act_normal(m, 4 * c, 1) for m in (1, 8, 32)}
    t0 = time.perf_counter()
    nbytes = 0
    layers = 0
    while True:
        for mat, n, k in synth.layer_shapes(c):
            w = synth.weight(1, layers, mat, n, k)
            parts = quant.quantize_sym(w, 4, 64)
            nbytes += 3 * (parts["codes"].nbytes + parts["scales"].nbytes)
            for m in (1, 8, 32):
                x = xs[m] if k == c else x4[m]
                ref.weight_only_ref(x, quant.W4_SYM, parts, 64)
        layers += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d layer(s) of the width-%d stack (6 matrices, w4g64), quantize + dequantize "
                      "+ fp64 product at M=1,8,32, %.1f s" % (layers, c, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phases", action="store_true", help="print per-phase timings to stderr")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library and this benchmark have no multi-GPU "
              "path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    # ---- 1.5B decode stack, w4g64
    C, NL = 2048, synth.RWKV7_SIZES["1.5B"][0]
    layers = [Layer(C, rq.RQ_W4_SYM, 64, gen, dev) for _ in range(NL)]
    wbytes = sum(L.weight_bytes() for L in layers)
    Ms = (1, 8, 32)
    xc = {m: f16_dev(synth.act_channel_1202(m, C), dev) for m in Ms}
    x4c = {m: f16_dev(synth.act_normal(m, 4 * C, 1), dev) for m in Ms}
    ys = {m: {name: torch.empty(m * (4 * C if name == "key" else C), dtype=torch.int16, device=dev)
              for name in ("r", "k", "v", "o", "key", "val")} for m in Ms}
    graphs = [capture(lambda m=m: decode_pass(layers, xc[m], x4c[m], ys[m], m, C)) for m in Ms]

    # ---- 7.2B prefill set, fp8, M = 256 (six copies: > 1 GiB of weights)
    C3, M3 = 4096, 256
    sets = []
    for _ in range(6):
        s = {}
        for mat, n, k in synth.layer_shapes(C3):
            wf = torch.randn(n, k, generator=gen, device=dev) * (1.0 / k ** 0.5)
            s[mat] = rq.quantize(wf, rq.RQ_FP8_E4M3_CH)
            del wf
        sets.append(s)
    xa = f16_dev(synth.act_normal(M3, C3, 3), dev)
    xa4 = f16_dev(synth.act_normal(M3, 4 * C3, 3, salt=1), dev)
    xq = torch.empty(M3 * C3, dtype=torch.uint8, device=dev)
    xq4 = torch.empty(M3 * 4 * C3, dtype=torch.uint8, device=dev)
    sx = torch.empty(M3, dtype=torch.float32, device=dev)
    sx4 = torch.empty(M3, dtype=torch.float32, device=dev)
    yp = torch.empty(M3 * 4 * C3, dtype=torch.int16, device=dev)

    def prefill():
        for s in sets:
            rq.rq_quantize_act(xa, M3, C3, C3, rq.RQ_FP8_E4M3_CH, xq, sx)
            for mat in (synth.MAT_R, synth.MAT_K, synth.MAT_V, synth.MAT_O, synth.MAT_KEY):
                rq.rq_gemm_fp8(xq, sx, M3, s[mat], yp, s[mat].n)
            rq.rq_quantize_act(xa4, M3, 4 * C3, 4 * C3, rq.RQ_FP8_E4M3_CH, xq4, sx4)
            rq.rq_gemm_fp8(xq4, sx4, M3, s[synth.MAT_VALUE], yp, C3)

    graphs.append(capture(prefill))
    flops = 6 * sum(2.0 * M3 * n * k for _, n, k in synth.layer_shapes(C3))

    per, wall = timed(graphs, args.steps, args.warmup)
    dec_ms = sum(per[:3])
    value = 3 * wbytes / (dec_ms * 1e-3) / 1e9
    fp8_tflops = flops / (per[3] * 1e-3) / 1e12
    if args.phases:
        for name, t, b in zip(("M=1", "M=8", "M=32"), per[:3], [wbytes] * 3):
            print("decode %s: %.3f ms, %.0f GB/s" % (name, t, b / t / 1e6), file=sys.stderr)
        print("prefill fp8 M=256: %.3f ms, %.1f TFLOP/s" % (per[3], fp8_tflops), file=sys.stderr)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "rwkv7-1.5B decode: 24 layers x (fused RKV, O, cmix key, cmix value), "
                               "int4 sym g64, M in {1,8,32}; plus rwkv7-7.2B fp8 prefill set at M=256",
                   "width": C, "layers": NL, "M": list(Ms), "weight_bytes_per_pass": wbytes,
                   "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4)},
        "fp8_gemm_m256": {"tflops": round(fp8_tflops, 1), "frac_of_peak": round(fp8_tflops / FP8_PEAK_TFLOPS, 4),
                          "ms": round(per[3], 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(C)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
