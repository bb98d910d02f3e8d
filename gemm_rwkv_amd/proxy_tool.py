"""RWKVQuant's coarse-to-fine proxy over every 2-D weight of a checkpoint.

    python -m gemm_rwkv_amd.proxy_tool model.safetensors [--K 4] [--tau-c 1.54] [--tau-f 30]
    python -m gemm_rwkv_amd.proxy_tool --synthetic 2048

Prints P_c, P_f and the scalar/vector routing of each tensor (RWKVQuant:
Quantizing the RWKV Family with Proxy Guided Hybrid of Scalar and Vector
Quantization -- machine-review page, pith_extraction.key_machinery: scalar
quantization only when P_c < tau_c and P_f < tau_f; tau_c = 1.54 and
tau_f = 30 reported for RWKV-7), computed by librq's rq_proxy on the host.
Checkpoints load through safetensors (no code is executed from the file);
--synthetic runs on the seeded N(0, 1/K) projections of one layer of the
given width.
"""

import argparse
import sys

from . import rq, synth


def _tensors(args):
    if args.synthetic:
        for mat, n, k in synth.layer_shapes(args.synthetic):
            yield "layer0.%s %dx%d" % (("R", "K", "V", "O", "cmix_key", "cmix_value")[mat], n, k), \
                synth.weight(0, 0, mat, n, k)
        return
    from safetensors.torch import load_file
    for name, t in load_file(args.path, device="cpu").items():
        if t.dim() == 2 and t.is_floating_point() and t.numel() >= 3:
            yield name, t


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("path", nargs="?")
    ap.add_argument("--synthetic", type=int, metavar="WIDTH")
    ap.add_argument("--K", type=int, default=4)
    ap.add_argument("--tau-c", type=float, default=1.54)
    ap.add_argument("--tau-f", type=float, default=30.0)
    args = ap.parse_args(argv)
    if not args.path and not args.synthetic:
        ap.error("give a .safetensors file or --synthetic WIDTH")
    counts = {"SQ": 0, "VQ": 0}
    print("%-48s %12s %12s %s" % ("tensor", "P_c", "P_f", "route"))
    for name, t in _tensors(args):
        try:
            pc, pf, _ = rq.rq_proxy(t, K=args.K)
        except rq.RqError as e:
            print("%-48s %s" % (name, e))
            continue
        r = rq.proxy_route(pc, pf, args.tau_c, args.tau_f)
        counts[r] += 1
        print("%-48s %12.6f %12.6f %s" % (name[:48], pc, pf, r))
    print("SQ %d, VQ %d" % (counts["SQ"], counts["VQ"]))
    return 0


if __name__ == "__main__":
    sys.exit(main())
