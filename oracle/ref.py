"""fp64 reference products and the pass/fail comparator (oracle).

Test infrastructure only.

The quantized-weight products compute exactly "dequantize, then multiply"
without materializing the dequantized copy ("RWKV-7 Quantization Toolkit",
opening line and Key Design: inference directly on quantized weights;
"RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang", summary: the kernel output
matches the offline dequantization).  So the reference is that plain
definition, in fp64:

    y_ref[m][n] = sum_k x_hat[m][k] * w_hat[n][k]
    B[m][n]     = sum_k |x_hat[m][k]| * |w_hat[n][k]|

with x_hat = x (fp16) for the weight-only paths, or the dequantized fp8/int8
activation codes for the W8A8/FP8 paths, and w_hat the dequantized weight.
The library's outputs are fp16 computed with fp32 accumulation; the accepted
error per element is ``|y - y_ref| <= 2e-3 * B + 1e-3`` and overall
``||y - y_ref||_2 <= 1e-3 * ||y_ref||_2``; any non-finite output fails.
"""

import numpy as np

from . import quant

ATOL = 1e-3
RTOL_B = 2e-3
RTOL_L2 = 1e-3


def matmul_ref(xhat, what):
    """fp64 product and magnitude bound: (y_ref [M][N], B [M][N])."""
    xhat = np.atleast_2d(np.asarray(xhat, dtype=np.float64))
    what = np.asarray(what, dtype=np.float64)
    if xhat.shape[1] != what.shape[1]:
        raise ValueError("inner dimensions differ")
    return xhat @ what.T, np.abs(xhat) @ np.abs(what).T


def weight_only_ref(x16, fmt, parts, group=0):
    """y_ref, B for fp16 activations x[M][K] against a quantized weight."""
    x = np.atleast_2d(np.asarray(x16, dtype=np.float16)).astype(np.float64)
    return matmul_ref(x, quant.dequant(fmt, parts, group))


def w8a8_ref(xq, sx, kind, fmt, parts):
    """y_ref, B for per-token quantized activations against a per-channel weight."""
    xhat = quant.dequant_rows(xq, sx, kind)
    return matmul_ref(xhat, quant.dequant(fmt, parts))


def int_acc_ref(xq, wq):
    """Exact integer accumulators sum_k xq[m][k] * wq[n][k] (int64)."""
    a = np.asarray(xq).view(np.int8).astype(np.int64)
    b = np.asarray(wq).view(np.int8).astype(np.int64)
    return a @ b.T


def compare(y, y_ref, bound):
    """Check fp16 outputs y against the fp64 reference.

    Returns (ok, info) with info = dict(max_ratio, rel_l2, nonfinite).
    ``max_ratio`` is max |y - y_ref| / (2e-3 * B + 1e-3); it must be <= 1.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (y.shape, y_ref.shape))
    nonfinite = int(np.count_nonzero(~np.isfinite(y)))
    err = np.abs(y - y_ref)
    tol = RTOL_B * bound + ATOL
    max_ratio = float(np.max(err / tol)) if err.size else 0.0
    nref = float(np.linalg.norm(y_ref))
    rel_l2 = float(np.linalg.norm(y - y_ref) / nref) if nref > 0 else float(np.linalg.norm(y - y_ref))
    ok = nonfinite == 0 and max_ratio <= 1.0 and rel_l2 <= RTOL_L2 if err.size else True
    return ok, {"max_ratio": max_ratio, "rel_l2": rel_l2, "nonfinite": nonfinite}
