"""Numerics of the int4 prefill GEMM on asymmetric superblocks, emulated on
the CPU against the oracle (no kernel runs here).

The kernel applies S_j and M_j in fp32 after the MFMA (per 32-group j:
S_j * sum(x u) - M_j * sum(x), nothing rounded below fp32).  A design that
dequantizes each weight to fp16 first, fma16(u, fp16(S_j), fp16(-M_j)),
errs by up to ~2^-11 * M_j per weight whatever the weight's size; on inputs
with massive channels over near-zero weights in groups with large offsets
that breaks the 1e-3 relative-L2 bound.  Both are emulated here on such an
input: the fp32 scheme must pass and the fp16 one must fail, which shows the
input exercises the difference."""

import numpy as np

from gemm_rwkv_amd import synth
from oracle import quant, ref


def _input(n=64, k=4096, m=8, seed=3):
    g = np.random.default_rng(seed)
    w = (g.uniform(-2.0, 0.1, (n, k)) / np.sqrt(k)).astype(np.float32)
    w[:, synth.massive_channels(k)] = 0.0
    return w, synth.act_massive(m, k, salt=seed)


def _group_params(parts):
    """S_j, M_j (fp64, exact) per 32-group [n][k/32] and the codes u [n][k]."""
    sc, mc = quant.unpack_sub(parts["sub"])
    n, nsb, _ = sc.shape
    d = parts["d"].astype(np.float64)[:, :, None]
    dmin = parts["dmin"].astype(np.float64)[:, :, None]
    S = (d * sc.astype(np.float64)).reshape(n, nsb * 8)
    M = (dmin * mc.astype(np.float64)).reshape(n, nsb * 8)
    u = quant.unpack_nibbles(parts["qs"]).astype(np.float64)
    return S, M, u


def _emulate_fp32_scaling(x, S, M, u):
    """sum over groups of fp32(S_j * sum_g(x u)) - fp32(M_j * sum_g(x)), in fp32."""
    m, k = x.shape
    x32 = x.astype(np.float32).reshape(m, k // 32, 32)
    u32 = u.astype(np.float32).reshape(-1, k // 32, 32)
    xu = np.einsum("mgk,ngk->mng", x32, u32).astype(np.float32)
    xs = x32.sum(axis=2, dtype=np.float32)
    acc = (S.astype(np.float32)[None] * xu - M.astype(np.float32)[None] * xs[:, None, :]).astype(np.float32)
    return acc.sum(axis=2, dtype=np.float32).astype(np.float16)


def _emulate_fp16_dequant(x, S, M, u):
    sh = np.repeat(S.astype(np.float16), 32, axis=1).astype(np.float64)
    mh = np.repeat((-M).astype(np.float16), 32, axis=1).astype(np.float64)
    w16 = (u * sh + mh).astype(np.float16)          # one rounding (fma)
    return (x.astype(np.float64) @ w16.astype(np.float64).T).astype(np.float16)


def test_fp32_scaling_meets_tolerance_where_fp16_dequant_fails():
    w, x = _input()
    parts = quant.quantize(w, quant.W4_ASYM_SB256, 32)
    S, M, u = _group_params(parts)
    assert np.all((u >= 0) & (u <= 15))
    # the emulated codes reproduce the oracle's dequantized weights exactly
    assert np.array_equal(np.repeat(S, 32, axis=1) * u - np.repeat(M, 32, axis=1),
                          quant.dequant(quant.W4_ASYM_SB256, parts))
    y_ref, b = ref.weight_only_ref(x, quant.W4_ASYM_SB256, parts, 32)
    ok32, info32 = ref.compare(_emulate_fp32_scaling(x, S, M, u), y_ref, b)
    ok16, info16 = ref.compare(_emulate_fp16_dequant(x, S, M, u), y_ref, b)
    assert ok32, info32
    assert not ok16, info16
