"""Helpers for the GPU parity tests: move oracle buffers to the device and
back as raw bytes, and wrap them in the binding's QWeight."""

import sys

import numpy as np
import torch

import gemm_rwkv_amd.rq as rq
from oracle import quant

GUARD = 4096  # bytes of sentinel margin around every output buffer
SENTINEL = 0xA5


def dev_bytes(a):
    """numpy array -> uint8 cuda tensor holding its bytes."""
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.reshape(-1).view(np.uint8).copy()).cuda()


def host(t, dtype, shape=None):
    a = t.detach().cpu().numpy().view(dtype)
    return a.reshape(shape) if shape is not None else a


def dev_f16(a):
    """fp16 numpy array -> cuda uint8 tensor of its bytes (use .data_ptr())."""
    return dev_bytes(np.asarray(a, dtype=np.float16))


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def qweight_from_oracle(fmt, group, parts, n, k):
    """QWeight whose device buffers hold the oracle's packed layout."""
    if fmt in (quant.W4_SYM, quant.W8_SYM):
        return rq.QWeight(fmt, group, n, k, dev_bytes(parts["codes"]), dev_bytes(parts["scales"]))
    if fmt in (quant.W6_SYM, quant.W5_SYM):
        return rq.QWeight(fmt, group, n, k, dev_bytes(parts["codes"]), dev_bytes(parts["scales"]),
                          None, dev_bytes(parts["hi"]))
    if fmt == quant.W4_ASYM_SB256:
        return rq.QWeight(fmt, 32, n, k, dev_bytes(parts["qs"]), dev_bytes(parts["d"]),
                          dev_bytes(parts["dmin"]), dev_bytes(parts["sub"]))
    if fmt in (quant.FP8_E4M3_CH, quant.I8_CH):
        return rq.QWeight(fmt, 0, n, k, dev_bytes(parts["codes"]), dev_bytes(parts["scales"]))
    if fmt in (quant.F16, quant.BF16):
        return rq.QWeight(fmt, 0, n, k, dev_bytes(parts["codes"]))
    raise ValueError(fmt)


def oracle_buffers(fmt, parts):
    """The oracle's packed buffers in the library's order (codes, scales, mins, sub)."""
    if fmt in (quant.W4_SYM, quant.W8_SYM):
        return {"codes": parts["codes"], "scales": parts["scales"]}
    if fmt in (quant.W6_SYM, quant.W5_SYM):
        return {"codes": parts["codes"], "scales": parts["scales"], "sub": parts["hi"]}
    if fmt == quant.W4_ASYM_SB256:
        return {"codes": parts["qs"], "scales": parts["d"], "mins": parts["dmin"], "sub": parts["sub"]}
    if fmt in (quant.FP8_E4M3_CH, quant.I8_CH):
        return {"codes": parts["codes"], "scales": parts["scales"]}
    return {"codes": parts["codes"]}


class Guarded:
    """An output buffer with sentinel-filled margins on both sides."""

    def __init__(self, nbytes):
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + nbytes]

    def ptr(self):
        return self.t.data_ptr()

    def check_guards(self):
        lo = self.buf[:GUARD]
        hi = self.buf[GUARD + self.nbytes:]
        assert bool((lo == SENTINEL).all()) and bool((hi == SENTINEL).all()), "write outside the output"


def say(*args):
    """Print what names the case before a GPU step, flushed."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def random_parts(fmt, group, n, k, g):
    """Seeded random packed buffers of a weight format, in the oracle's layout
    (inputs for products; every byte pattern is a valid code).  Scales are
    fp16 in [2^-10, 2^-9); fp16 / bf16 weights are N(0, 1/k)."""
    def scales(cols):
        return (g.integers(0, 1024, (n, cols)) | (5 << 10)).astype(np.uint16).view(np.float16)
    if fmt == quant.W4_ASYM_SB256:
        nsb = k // 256
        return {"qs": g.integers(0, 256, (n, k // 2), dtype=np.uint8), "d": scales(nsb), "dmin": scales(nsb),
                "sub": g.integers(0, 256, (n, nsb, 12), dtype=np.uint8)}
    if fmt == quant.F16:
        return {"codes": (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float16)}
    if fmt == quant.BF16:
        f = (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
        return {"codes": (f.view(np.uint32) >> 16).astype(np.uint16)}   # truncated to bf16
    nbytes = k if fmt == quant.W8_SYM else k // 2
    parts = {"codes": g.integers(0, 256, (n, nbytes), dtype=np.uint8), "scales": scales(k // group)}
    if fmt == quant.W6_SYM:
        parts["hi"] = g.integers(0, 1 << 16, (n, k // 8)).astype(np.uint16)
    elif fmt == quant.W5_SYM:
        parts["hi"] = g.integers(0, 256, (n, k // 8), dtype=np.uint8)
    return parts


def rows_of(parts, rows):
    """The same buffers restricted to the given weight rows."""
    return {name: arr[rows] for name, arr in parts.items()}
