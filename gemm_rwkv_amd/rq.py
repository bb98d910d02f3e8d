"""ctypes binding of librq (include/rq.h), argument marshalling only.

Every function keeps the C name and takes torch tensors where the C function
takes device pointers; the tensors are plain device memory (PyTorch supplies
allocation and the current stream).  All computation happens in librq's HIP
kernels.  Loading fails loudly if ``librq.so`` has not been built.
"""

import ctypes
import os

import torch

# RQ_LIBRARY selects another build of the same library (the sanitized one)
_LIB_PATH = os.environ.get("RQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "librq.so")

RQ_OK = 0
RQ_ERR_NULL = -1
RQ_ERR_SHAPE = -2
RQ_ERR_ALIGN = -3
RQ_ERR_FORMAT = -4
RQ_ERR_NONFINITE = -5
RQ_ERR_RANGE = -6
RQ_ERR_HIP = -7
RQ_ERR_ALIAS = -8
RQ_ERR_SCRATCH = -9
RQ_ERR_DEGENERATE = -10
RQ_PROXY_MAX_K = 16

RQ_W8_SYM = 1
RQ_W4_SYM = 2
RQ_W4_ASYM_SB256 = 3
RQ_FP8_E4M3_CH = 4
RQ_I8_CH = 5
RQ_F16 = 6
RQ_W5_SYM = 7
RQ_W6_SYM = 8
RQ_BF16 = 9

# every symbol include/rq.h declares
EXPORTS = (
    "rq_abi_version", "rq_status_str", "rq_qweight_bytes", "rq_quantize_rtn",
    "rq_gemv_w4g16", "rq_gemv_w4g32", "rq_gemv_w4g64", "rq_gemv_w8g16", "rq_gemv_w8g32",
    "rq_gemv_w8g64", "rq_gemv_w4sb256", "rq_gemv_f16", "rq_gemm_small_m", "rq_fused_rkv",
    "rq_quantize_act", "rq_gemm_fp8", "rq_gemm_int8", "rq_gemm_int8_acc", "rq_host_convert",
    "rq_gemm_w4", "rq_quantize_aw", "rq_workspace_bytes", "rq_gemm_small_m_noalloc", "rq_stream_read",
    "rq_proxy", "rq_plan_small_m",
)

# rq_plan.kernel
RQ_PLAN_NONE, RQ_PLAN_STREAMING, RQ_PLAN_TWO_RANGES, RQ_PLAN_STREAMED_X, RQ_PLAN_PHASED, RQ_PLAN_FIRST = range(6)


class RqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, status_str(status), status))


class _QW(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("group", ctypes.c_int32), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("mins", ctypes.c_void_p), ("sub", ctypes.c_void_p)]


class _Plan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in ("kernel", "split", "chunks_per_slice", "chunks_per_wave",
                                                    "waves_per_tile", "tiles_per_workgroup", "workgroups",
                                                    "threads")] + \
               [("lds_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded librq (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("librq.so is not built (run gemm_rwkv_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        qp = ctypes.POINTER(_QW)
        sig = {
            "rq_abi_version": ([], i32),
            "rq_status_str": ([i32], ctypes.c_char_p),
            "rq_qweight_bytes": ([i32, i32, i64, i64] + [ctypes.POINTER(ctypes.c_size_t)] * 4, i32),
            "rq_quantize_rtn": ([vp, qp, vp], i32),
            "rq_quantize_aw": ([vp, vp, qp, vp], i32),
            "rq_gemm_small_m": ([vp, i64, i64, qp, vp, i64, vp, sz, vp], i32),
            "rq_gemm_w4": ([vp, i64, i64, qp, vp, i64, vp, sz, vp], i32),
            "rq_fused_rkv": ([vp, vp, vp, i64, i64, qp, qp, qp, vp, vp, vp, i64, vp, sz, vp], i32),
            "rq_quantize_act": ([vp, i64, i64, i64, i32, vp, vp, vp], i32),
            "rq_gemm_fp8": ([vp, vp, i64, qp, vp, i64, vp, sz, vp], i32),
            "rq_gemm_int8": ([vp, vp, i64, qp, vp, i64, vp, sz, vp], i32),
            "rq_gemm_int8_acc": ([vp, i64, qp, vp, vp, sz, vp], i32),
            "rq_workspace_bytes": ([], sz),
            "rq_gemm_small_m_noalloc": ([vp, i64, i64, qp, vp, i64, vp], i32),
            "rq_stream_read": ([vp, sz, vp, vp], i32),
            "rq_proxy": ([vp, i64, i32, vp, vp, vp, vp], i32),
            "rq_host_convert": ([i32, vp, vp, i64], i32),
            "rq_plan_small_m": ([qp, i64, i64, sz, ctypes.POINTER(_Plan)], i32),
        }
        for name in ("rq_gemv_w4g16", "rq_gemv_w4g32", "rq_gemv_w4g64", "rq_gemv_w8g16",
                     "rq_gemv_w8g32", "rq_gemv_w8g64", "rq_gemv_w4sb256", "rq_gemv_f16"):
            sig[name] = ([vp, qp, vp, vp, sz, vp], i32)
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_str(status):
    return lib().rq_status_str(int(status)).decode()


def _check(st, where):
    if st != RQ_OK:
        raise RqError(st, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_default_ws = {}


def default_workspace(device=None):
    """The binding's default workspace on a device: a uint8 tensor of
    rq_workspace_bytes(), allocated on first use and kept.  It is shared by
    every call that passes no workspace of its own, so such calls must not
    run concurrently.  It is zero-filled (its first 64 KiB are the split
    counters, which every call leaves at zero) and synchronized before first
    use.  Allocating it while a graph is being captured is refused: call this
    once before capturing."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else torch.device(device).index or 0)
    t = _default_ws.get(dev.index)
    if t is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("rq: allocate the default workspace before graph capture "
                               "(call gemm_rwkv_amd.rq.default_workspace() first)")
        t = torch.zeros(lib().rq_workspace_bytes(), dtype=torch.uint8, device=dev)
        # the split counters at its head must read zero from any stream
        torch.cuda.synchronize(dev)
        _default_ws[dev.index] = t
    return t


def _ws(ws):
    """(pointer, bytes) of a workspace argument: None = the default
    workspace, False = none, or a uint8 device tensor."""
    if ws is False:
        return None, 0
    if ws is None:
        if not torch.cuda.is_available():
            return None, 0
        ws = default_workspace()
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _stream(stream):
    if stream is None:
        # without a GPU (argument checks only) there is no current stream
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------
# quantized weights
# --------------------------------------------------------------------------


def rq_qweight_bytes(fmt, group, n, k):
    """(codes, scales, mins, sub) byte sizes; raises RqError on a bad shape."""
    out = [ctypes.c_size_t() for _ in range(4)]
    st = lib().rq_qweight_bytes(fmt, group, n, k, *[ctypes.byref(o) for o in out])
    _check(st, "rq_qweight_bytes")
    return tuple(o.value for o in out)


class QWeight:
    """A quantized weight: format, group, n, k and its device buffers (uint8
    torch tensors sized by rq_qweight_bytes; unused ones are None)."""

    def __init__(self, fmt, group, n, k, codes, scales=None, mins=None, sub=None):
        self.format, self.group, self.n, self.k = int(fmt), int(group), int(n), int(k)
        self.codes, self.scales, self.mins, self.sub = codes, scales, mins, sub

    @classmethod
    def empty(cls, fmt, group, n, k, device="cuda"):
        sizes = rq_qweight_bytes(fmt, group, n, k)
        bufs = [torch.empty(max(s, 1), dtype=torch.uint8, device=device) if s or i == 0 else None
                for i, s in enumerate(sizes)]
        return cls(fmt, group, n, k, *bufs)

    def desc(self):
        return _QW(self.format, self.group, self.n, self.k, _ptr(self.codes), _ptr(self.scales),
                   _ptr(self.mins), _ptr(self.sub))

    def nbytes(self):
        return sum(rq_qweight_bytes(self.format, self.group, self.n, self.k))

    def buffers(self):
        """name -> uint8 tensor of the used buffers (trimmed to their sizes)."""
        sizes = rq_qweight_bytes(self.format, self.group, self.n, self.k)
        out = {}
        for name, t, s in zip(("codes", "scales", "mins", "sub"),
                              (self.codes, self.scales, self.mins, self.sub), sizes):
            if s:
                out[name] = t[:s]
        return out


def rq_quantize_rtn(w, out, stream=None):
    """Quantize fp32 device weights w[n][k] into the QWeight ``out`` (synchronizes)."""
    d = out.desc()
    st = lib().rq_quantize_rtn(_ptr(w), ctypes.byref(d), _stream(stream))
    _check(st, "rq_quantize_rtn")
    return out


def rq_quantize_aw(w, act_sq, out, stream=None):
    """Activation-weighted quantization of fp32 device weights w[n][k] with
    per-channel E[x^2] importances act_sq[k] (fp32, device) into ``out``
    (synchronizes)."""
    d = out.desc()
    st = lib().rq_quantize_aw(_ptr(w), _ptr(act_sq), ctypes.byref(d), _stream(stream))
    _check(st, "rq_quantize_aw")
    return out


def quantize(w, fmt, group=0, stream=None):
    """Allocate a QWeight for fp32 device weights w and fill it with rq_quantize_rtn."""
    n, k = w.shape
    q = QWeight.empty(fmt, group, n, k, device=w.device)
    return rq_quantize_rtn(w, q, stream)


def quantize_aw(w, act_sq, fmt, group=0, stream=None):
    """Allocate a QWeight for fp32 device weights w and fill it with rq_quantize_aw."""
    n, k = w.shape
    q = QWeight.empty(fmt, group, n, k, device=w.device)
    return rq_quantize_aw(w, act_sq, q, stream)


# --------------------------------------------------------------------------
# products
# --------------------------------------------------------------------------


def _gemv(name):
    def f(x, w, y, stream=None, ws=None):
        d = w.desc()
        st = getattr(lib(), name)(_ptr(x), ctypes.byref(d), _ptr(y), *_ws(ws), _stream(stream))
        _check(st, name)
        return y
    f.__name__ = name
    f.__doc__ = "M=1 product y[n] = sum_k x[k] W_hat[n][k] (librq %s)." % name
    return f


rq_gemv_w4g16 = _gemv("rq_gemv_w4g16")
rq_gemv_w4g32 = _gemv("rq_gemv_w4g32")
rq_gemv_w4g64 = _gemv("rq_gemv_w4g64")
rq_gemv_w8g16 = _gemv("rq_gemv_w8g16")
rq_gemv_w8g32 = _gemv("rq_gemv_w8g32")
rq_gemv_w8g64 = _gemv("rq_gemv_w8g64")
rq_gemv_w4sb256 = _gemv("rq_gemv_w4sb256")
rq_gemv_f16 = _gemv("rq_gemv_f16")

GEMV_ENTRY = {
    (RQ_W4_SYM, 16): rq_gemv_w4g16, (RQ_W4_SYM, 32): rq_gemv_w4g32, (RQ_W4_SYM, 64): rq_gemv_w4g64,
    (RQ_W8_SYM, 16): rq_gemv_w8g16, (RQ_W8_SYM, 32): rq_gemv_w8g32, (RQ_W8_SYM, 64): rq_gemv_w8g64,
    (RQ_W4_ASYM_SB256, 32): rq_gemv_w4sb256, (RQ_F16, 0): rq_gemv_f16,
}


def rq_gemm_small_m(x, m, ldx, w, y, ldy, stream=None, ws=None):
    d = w.desc()
    st = lib().rq_gemm_small_m(_ptr(x), m, ldx, ctypes.byref(d), _ptr(y), ldy, *_ws(ws), _stream(stream))
    _check(st, "rq_gemm_small_m")
    return y


def rq_plan_small_m(w, m, ldx=None, ws_bytes=None):
    """The launch rq_gemm_small_m would make (host only): a dict of rq_plan's
    fields.  ws_bytes defaults to rq_workspace_bytes(); 0 means no
    workspace.  w may be a QWeight or a (format, group, n, k) tuple."""
    if isinstance(w, tuple):
        fmt, group, n, k = w
        # descriptor of 256-aligned placeholder addresses: the planner reads
        # the shapes only
        d = _QW(fmt, group, n, k, 256, 256, 256, 256)
    else:
        d = w.desc()
    if ldx is None:
        ldx = d.k + (8 - d.k % 8) % 8
    if ws_bytes is None:
        ws_bytes = lib().rq_workspace_bytes()
    p = _Plan()
    st = lib().rq_plan_small_m(ctypes.byref(d), m, ldx, ws_bytes, ctypes.byref(p))
    _check(st, "rq_plan_small_m")
    return {name: getattr(p, name) for name, _ in _Plan._fields_}


def rq_gemm_small_m_noalloc(x, m, ldx, w, y, ldy, stream=None):
    """rq_gemm_small_m with the library's static scratch (allocates nothing)."""
    d = w.desc()
    st = lib().rq_gemm_small_m_noalloc(_ptr(x), m, ldx, ctypes.byref(d), _ptr(y), ldy, _stream(stream))
    _check(st, "rq_gemm_small_m_noalloc")
    return y


def rq_gemm_w4(x, m, ldx, w, y, ldy, stream=None, ws=None):
    d = w.desc()
    st = lib().rq_gemm_w4(_ptr(x), m, ldx, ctypes.byref(d), _ptr(y), ldy, *_ws(ws), _stream(stream))
    _check(st, "rq_gemm_w4")
    return y


def rq_fused_rkv(xr, xk, xv, m, ldx, wr, wk, wv, yr, yk, yv, ldy, stream=None, ws=None):
    ds = [wr.desc(), wk.desc(), wv.desc()]
    st = lib().rq_fused_rkv(_ptr(xr), _ptr(xk), _ptr(xv), m, ldx, *[ctypes.byref(d) for d in ds],
                            _ptr(yr), _ptr(yk), _ptr(yv), ldy, *_ws(ws), _stream(stream))
    _check(st, "rq_fused_rkv")
    return yr, yk, yv


def rq_quantize_act(x, m, k, ldx, fmt, xq, sx, stream=None):
    st = lib().rq_quantize_act(_ptr(x), m, k, ldx, fmt, _ptr(xq), _ptr(sx), _stream(stream))
    _check(st, "rq_quantize_act")
    return xq, sx


def rq_gemm_fp8(xq, sx, m, w, y, ldy, stream=None, ws=None):
    d = w.desc()
    st = lib().rq_gemm_fp8(_ptr(xq), _ptr(sx), m, ctypes.byref(d), _ptr(y), ldy, *_ws(ws), _stream(stream))
    _check(st, "rq_gemm_fp8")
    return y


def rq_gemm_int8(xq, sx, m, w, y, ldy, stream=None, ws=None):
    d = w.desc()
    st = lib().rq_gemm_int8(_ptr(xq), _ptr(sx), m, ctypes.byref(d), _ptr(y), ldy, *_ws(ws), _stream(stream))
    _check(st, "rq_gemm_int8")
    return y


def rq_gemm_int8_acc(xq, m, w, acc, stream=None, ws=None):
    d = w.desc()
    st = lib().rq_gemm_int8_acc(_ptr(xq), m, ctypes.byref(d), _ptr(acc), *_ws(ws), _stream(stream))
    _check(st, "rq_gemm_int8_acc")
    return acc


def rq_stream_read(buf, nbytes, sink, stream=None):
    """Read-only stream over nbytes of the device buffer buf (measurement aid)."""
    _check(lib().rq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "rq_stream_read")


def rq_proxy(w, K=4, v=None):
    """RWKVQuant's coarse-to-fine proxy of one weight tensor on the host:
    (P_c, P_f, [M_2..M_K]).  w: anything numpy can view as float32 (a CPU or
    GPU tensor is copied to host memory first); v: K - 1 weights for
    k = 2..K, None for 1/k!."""
    import numpy as np
    if isinstance(w, torch.Tensor):
        w = w.detach().to("cpu", torch.float32).numpy()
    a = np.ascontiguousarray(np.asarray(w, dtype=np.float32).ravel())
    vv = None
    if v is not None:
        vv = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
        if vv.size != K - 1:
            raise ValueError("v needs K - 1 weights (k = 2..K)")
    pc, pf = ctypes.c_double(), ctypes.c_double()
    mk = np.zeros(max(K - 1, 1), dtype=np.float64)
    _check(lib().rq_proxy(a.ctypes.data, a.size, int(K), None if vv is None else vv.ctypes.data,
                          ctypes.addressof(pc), ctypes.addressof(pf), mk.ctypes.data), "rq_proxy")
    return pc.value, pf.value, mk[:K - 1]


def proxy_route(pc, pf, tau_c=1.54, tau_f=30.0):
    """The pages' routing: scalar quantization ("SQ") only when P_c < tau_c
    and P_f < tau_f, else vector quantization ("VQ"); defaults are the
    thresholds reported for RWKV-7."""
    return "SQ" if (pc < tau_c and pf < tau_f) else "VQ"


def rq_workspace_bytes():
    return int(lib().rq_workspace_bytes())


def rq_host_convert(kind, values):
    """Host-side run of the library's fp64 -> fp16 / fp32 / e4m3fn conversions."""
    import numpy as np
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.empty(v.shape, dtype={0: np.uint16, 1: np.uint32, 2: np.uint8}[kind])
    st = lib().rq_host_convert(kind, v.ctypes.data, out.ctypes.data, v.size)
    _check(st, "rq_host_convert")
    return out
