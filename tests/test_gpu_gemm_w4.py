"""GPU parity of rq_gemm_w4 (prefill products on symmetric int4 codes, any m)
against the CPU oracle: fp16 outputs within |y - y_ref| <= 2e-3*B + 1e-3 and
relative L2 <= 1e-3 (oracle.ref.compare), and bit-exact where every product
and sum is an integer."""

import numpy as np
import pytest
import torch

import gemm_rwkv_amd.rq as rq
from gpu_helpers import SENTINEL, Guarded, dev_f16, host, qweight_from_oracle, say
from oracle import quant, ref

pytestmark = pytest.mark.gpu


def _run(qw, x, m, ldx, n, ldy=None):
    ldy = ldy or n + (3 if n % 2 else 8)
    y = Guarded(2 * max(m, 1) * ldy)
    say("gemm_w4", "group", qw.group, "m", m, "n", n, "k", qw.k, "ldx", ldx)
    rq.rq_gemm_w4(dev_f16(x), m, ldx, qw, y.ptr(), ldy)
    torch.cuda.synchronize()
    y.check_guards()
    return host(y.t, np.float16)[: m * ldy].reshape(m, ldy)[:, :n]


@pytest.mark.parametrize("group", [64, 32, 16])
@pytest.mark.parametrize("n,k,m", [
    # 64 x 64 tiles: one k block, ragged m and n; three blocks (the whole
    # ring once); nine blocks; a single row
    (100, 128, 37), (257, 384, 130), (300, 1152, 100), (64, 256, 1),
    # m <= 64: 64 x 128 tiles of eight waves (257 column tiles); 64 x 256
    # tiles of four waves (257 column tiles); ragged n
    (32770, 128, 50), (65540, 128, 60),
    # 128 x 128 tiles of eight waves (2 x 128), ragged m and n, two blocks
    (16300, 256, 250),
    # 64 x 64 tiles (4 x 65) over 32 k blocks, ragged m and n
    (4100, 4096, 200),
    # 128 x 256 tiles of eight waves (8 x 33), ragged m and n
    (8200, 128, 1000),
    # K split: 64 x 64 tiles in 2 slices of 8 blocks; 128 x 256 tiles in 8
    # slices of 8 blocks; ragged m and n
    (300, 2048, 70), (4000, 8192, 250)])
def test_gemm_w4_parity(group, n, k, m):
    g = np.random.default_rng(n + k + m + group)
    w = (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    parts = quant.quantize(w, quant.W4_SYM, group)
    qw = qweight_from_oracle(quant.W4_SYM, group, parts, n, k)
    ldx = k + 8
    x = g.standard_normal((m, ldx)).astype(np.float16)
    y = _run(qw, x, m, ldx, n)
    y_ref, b = ref.weight_only_ref(x[:, :k], quant.W4_SYM, parts, group)
    ok, info = ref.compare(y, y_ref, b)
    assert ok, info


@pytest.mark.parametrize("n,k,m", [
    # 64 x 64 tiles, one superblock (two k blocks); ragged m and n
    (100, 256, 37), (257, 768, 130),
    # 64 x 128 tiles of eight waves (m <= 64); 128 x 128 tiles of eight waves
    (32770, 256, 50), (16300, 512, 250),
    # K = 10240 (the width-2560 cmix value input) split in 8 slices of 10
    # blocks, on 64 x 128 and 64 x 64 tiles; 18 blocks split 9 + 9, so a
    # slice boundary falls inside a superblock; ragged m and n
    (2560, 10240, 100), (1000, 10240, 70), (300, 2304, 70)])
def test_gemm_w4_sb256_parity(n, k, m):
    g = np.random.default_rng(n + k + m + 7)
    w = (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    parts = quant.quantize(w, quant.W4_ASYM_SB256, 32)
    qw = qweight_from_oracle(quant.W4_ASYM_SB256, 32, parts, n, k)
    ldx = k + 8
    x = g.standard_normal((m, ldx)).astype(np.float16)
    y = _run(qw, x, m, ldx, n)
    y_ref, b = ref.weight_only_ref(x[:, :k], quant.W4_ASYM_SB256, parts, 32)
    ok, info = ref.compare(y, y_ref, b)
    assert ok, info


def test_gemm_w4_sb256_integer_exact():
    """d = dmin = 1 with sub-codes sc = 1, mc = 8 give S_j = 1 and M_j = 8, so
    w = u - 8 is exact in fp16 and every sum is an integer: the output equals
    the integer product exactly."""
    g = np.random.default_rng(11)
    n, k, m = 96, 512, 70
    u = g.integers(0, 16, (n, k))
    nsb = k // 256
    parts = {"qs": quant.pack_nibbles(u),
             "d": np.ones((n, nsb), np.float16), "dmin": np.ones((n, nsb), np.float16),
             "sub": quant.pack_sub(np.ones((n, nsb, 8), np.uint8), np.full((n, nsb, 8), 8, np.uint8))}
    qw = qweight_from_oracle(quant.W4_ASYM_SB256, 32, parts, n, k)
    x = g.integers(-1, 2, (m, k)).astype(np.float16)
    y = _run(qw, x, m, k, n)
    exact = x.astype(np.int64) @ (u - 8).astype(np.int64).T
    assert np.abs(exact).max() <= 2048
    assert np.array_equal(y.astype(np.float64), exact.astype(np.float64))


@pytest.mark.parametrize("group", [64, 16])
def test_gemm_w4_integer_exact(group):
    """A code of +-7 in every group gives scale 1 exactly, so w = q is exact in
    fp16 and, with x in {-1, 0, 1}, every product and partial sum is an
    integer below 2^24: the output equals the integer product exactly."""
    g = np.random.default_rng(group)
    n, k, m = 200, 256, 70
    q = g.integers(-3, 4, (n, k))
    q[:, ::group] = np.where(g.random((n, k // group)) < 0.5, -7, 7)
    parts = quant.quantize(q.astype(np.float32), quant.W4_SYM, group)
    assert np.all(parts["scales"] == np.float16(1.0))
    qw = qweight_from_oracle(quant.W4_SYM, group, parts, n, k)
    x = g.integers(-1, 2, (m, k)).astype(np.float16)
    y = _run(qw, x, m, k, n)
    exact = x.astype(np.int64) @ q.astype(np.int64).T
    assert np.abs(exact).max() <= 2048
    assert np.array_equal(y.astype(np.float64), exact.astype(np.float64))


def test_gemm_w4_deterministic_and_empty():
    g = np.random.default_rng(3)
    n, k, m = 300, 512, 90
    w = (g.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    parts = quant.quantize(w, quant.W4_SYM, 64)
    qw = qweight_from_oracle(quant.W4_SYM, 64, parts, n, k)
    x = g.standard_normal((m, k)).astype(np.float16)
    y1 = _run(qw, x, m, k, n)
    y2 = _run(qw, x, m, k, n)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    # m == 0 touches nothing
    y = Guarded(64)
    rq.rq_gemm_w4(dev_f16(x), 0, k, qw, y.ptr(), n)
    torch.cuda.synchronize()
    assert bool((y.buf == SENTINEL).all())


def _sb256_adversarial(n, k, m, seed):
    """Superblock weights with large offsets and near-cancelling values:
    w ~ U(-2, 0.1)/sqrt(k) (each group's minimum sets M_j ~ 2/sqrt(k) while
    S_j ~ M_j / 14), and zero weights on the 8 massive activation channels, so
    their dequantized weights S_j q - M_j are near zero while x there is ~300."""
    from gemm_rwkv_amd import synth
    g = np.random.default_rng(seed)
    w = (g.uniform(-2.0, 0.1, (n, k)) / np.sqrt(k)).astype(np.float32)
    w[:, synth.massive_channels(k)] = 0.0
    x = synth.act_massive(m, k, salt=seed)
    return w, x


@pytest.mark.parametrize("n,k,m", [(2560, 16384, 64), (2560, 16384, 16), (1000, 10240, 130)])
def test_sb256_adversarial(n, k, m):
    w, x = _sb256_adversarial(n, k, m, seed=n + m)
    parts = quant.quantize(w, quant.W4_ASYM_SB256, 32)
    qw = qweight_from_oracle(quant.W4_ASYM_SB256, 32, parts, n, k)
    y = _run(qw, x, m, k, n)
    y_ref, b = ref.weight_only_ref(x, quant.W4_ASYM_SB256, parts, 32)
    ok, info = ref.compare(y, y_ref, b)
    print("sb256 adversarial", n, k, m, info, flush=True)
    assert ok, info
