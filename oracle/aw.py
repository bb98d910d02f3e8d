"""Activation-weighted (AW) scale search for the symmetric and superblock
formats (oracle).

Test infrastructure only: tests, the smoke check and bench's cpu_baseline leg
may call this module; the GPU library never does.

The rwkv-quant news article ("rwkv-quant: uma matriz em bf16 elimina 39% das
perdas na quantização do RWKV-7 2.9B", section "Dois presets e seis tamanhos")
says that in both presets the scale and offset of each group are chosen by a
search weighted by E[x^2], the mean square of the channel's input activation;
section "Onde o 2.9B quebra" reports that without that weighting 4-bit o_proj
breaks the 2.9B model.  The article gives neither the search grid nor a tie
rule.  Readings used here (the library implements the same):

* Objective, per group: err = sum_k a_k (w_k - w_hat_k)^2 with a_k = E[x^2] of
  input channel k (a nonnegative fp32 vector of length K).
* Candidates: AW_STEPS = 16 shrink steps t = 0..15 with factor f_t = 1 - t/32
  (exact in fp64).  Symmetric: s_t = fp16((absmax / Q) * f_t), codes the RTN
  codes of that stored scale.  Superblocks: both ends of the group's RTN range
  scaled toward zero, lo_t = lo * f_t, hi_t = hi * f_t, s_t = (hi_t - lo_t) / 15,
  m_t = 0 - lo_t, u = clamp(RNE((w + m_t) / s_t), 0, 15), w_hat = s_t u - m_t.
  Step 0 is plain RTN.
* Choice: the smallest t whose err is at most (1 + 2^-40) times the smallest
  err.  The factor makes the choice independent of the order in which err is
  summed (the library sums in a different order), and among equal errors the
  least shrunk scale wins.
* Superblocks: the chosen (s_j, -lo_j) of each group then go through the RTN
  superblock step unchanged (d, dmin, 6-bit sub-codes, codes against the
  effective S_j and M_j); the search itself uses the unquantized s_t and m_t.
* Every code, scale and error term is a fixed sequence of IEEE fp64
  operations: (w - q*s), its square, times a, as written below.

Parity of the grid and the tie rule is unpinned by the pages (they give
neither); tests pin this specification: the step-0 case reduces to RTN, zero
importance gives RTN, the weighted error never exceeds RTN's, the choice
matches an exact rational brute force on small groups, and on activations with
massive channels AW lowers the output error against RTN.
"""

import numpy as np

from . import codecs, quant

AW_STEPS = 16
AW_TIE = 2.0 ** -40


def _factors():
    return [1.0 - t / 32.0 for t in range(AW_STEPS)]


def _check_importance(a, k):
    a = np.asarray(a, dtype=np.float32)
    if a.shape != (k,):
        raise ValueError("importance must have shape (K,)")
    if not np.all(np.isfinite(a)) or np.any(a < 0):
        raise ValueError("importance must be finite and nonnegative")
    return a.astype(np.float64)


def choose(err):
    """Index of the chosen candidate along axis 0 of err[T][...]: the smallest
    t with err[t] <= (1 + AW_TIE) * min_t err[t]."""
    emin = np.min(err, axis=0)
    thr = emin * (1.0 + AW_TIE)
    ok = err <= thr[None]
    return np.argmax(ok, axis=0)   # first True


def _sym_codes(wd, s, qmax):
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(wd / s), -qmax, qmax)
    return np.where(s == 0.0, 0.0, q)


def quantize_sym_aw(w, a, bits, group):
    """AW search for the symmetric format; returns quantize_sym's dict plus
    ``t`` (chosen step per (row, group)) and ``err`` (the candidates' errors)."""
    w = np.asarray(w, dtype=np.float32)
    quant._check_finite(w)
    n, k = w.shape
    quant.check_sym_shape(bits, group, k)
    ad = _check_importance(a, k).reshape(1, k // group, group)
    qmax = quant._qmax(bits)
    wd = w.astype(np.float64).reshape(n, k // group, group)
    base = np.max(np.abs(wd), axis=2) / float(qmax)
    s16 = []
    err = []
    for f in _factors():
        st16 = codecs.f16_encode(base * f)
        if not np.all(np.isfinite(st16)):
            raise OverflowError("fp16 scale overflow")
        s = st16.astype(np.float64)[:, :, None]
        q = _sym_codes(wd, s, qmax)
        d = wd - q * s
        err.append(np.sum(ad * (d * d), axis=2))
        s16.append(st16)
    err = np.stack(err)
    t = choose(err)
    s16 = np.take_along_axis(np.stack(s16), t[None], axis=0)[0]
    s = s16.astype(np.float64)[:, :, None]
    q = _sym_codes(wd, s, qmax).astype(np.int8).reshape(n, k)
    out = quant.sym_parts(q, s16, bits)
    out["t"] = t
    out["err"] = err
    return out


def quantize_sb256_aw(w, a):
    """AW search for the asymmetric superblocks; returns quantize_sb256's
    dict plus ``t`` (chosen step per group) and ``err``."""
    w = np.asarray(w, dtype=np.float32)
    quant._check_finite(w)
    n, k = w.shape
    if k % quant.SB:
        raise ValueError("K must be a multiple of 256")
    nsb = k // quant.SB
    ad = _check_importance(a, k).reshape(1, nsb, quant.SB_NGROUPS, quant.SB_GROUP)
    wd = w.astype(np.float64).reshape(n, nsb, quant.SB_NGROUPS, quant.SB_GROUP)
    hi = np.max(wd, axis=3)
    lo = quant._group_low(wd)
    ss, ms, err = [], [], []
    for f in _factors():
        lo_t = lo * f
        hi_t = hi * f
        s = (hi_t - lo_t) / 15.0
        s = np.where(s == 0.0, 0.0, s)
        m = 0.0 - lo_t
        with np.errstate(divide="ignore", invalid="ignore"):
            u = np.clip(np.rint((wd + m[..., None]) / s[..., None]), 0, 15)
        u = np.where(s[..., None] == 0.0, 0.0, u)
        d = wd - (s[..., None] * u - m[..., None])
        err.append(np.sum(ad * (d * d), axis=3))
        ss.append(s)
        ms.append(m)
    err = np.stack(err)
    t = choose(err)
    s = np.take_along_axis(np.stack(ss), t[None], axis=0)[0]
    neglo = np.take_along_axis(np.stack(ms), t[None], axis=0)[0]
    out = quant.sb256_from_group_params(wd, s, neglo)
    out["t"] = t
    out["err"] = err
    return out


def quantize_aw(w, a, fmt, group=0):
    """AW quantization of fp32 W[N][K] with importance a[K] into ``fmt``."""
    if fmt in quant.SYM_BITS:
        return quantize_sym_aw(w, a, quant.SYM_BITS[fmt], group)
    if fmt == quant.W4_ASYM_SB256:
        return quantize_sb256_aw(w, a)
    raise ValueError("AW search covers the symmetric and superblock formats")
