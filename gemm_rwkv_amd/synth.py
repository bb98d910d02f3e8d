"""Seeded synthetic inputs with the shapes of RWKV-7 projection layers.

This module only draws random numbers and lays them out; it holds none of the
quantization or product arithmetic, so both the GPU tests and the CPU oracle
can take their inputs from it.

Shapes (a matrix is W[N][K], N outputs, K inputs; C is the model width):
    R, K, V, O projections   [C][C]
    cmix key                 [4C][C]
    cmix value               [C][4C]
    head (vocab 65536)       [65536][C]
Model sizes are the RWKV-7 table in the rwkv-quant news article ("Dois presets
e seis tamanhos": 0.1B 12 x 768, 1.5B 24 x 2048, 2.9B 32 x 2560, 7.2B 32 x 4096,
13.3B 61 x 4096).

Weights are fp32 ~ N(0, 1/K).  Activations are fp16 ~ N(0, 1), optionally with
the "massive channels" the article reports ("Onde o 2.9B quebra": channel 1202
dominates the 1.5B input; on the 2.9B eight channels, channel 517 among them,
hold 98% of the energy).
"""

import numpy as np

# matrix ids used in seed keys
MAT_R, MAT_K, MAT_V, MAT_O, MAT_KEY, MAT_VALUE, MAT_HEAD = range(7)
MAT_NAMES = ("r", "k", "v", "o", "cmix_key", "cmix_value", "head")

RWKV7_SIZES = {  # name: (layers, width)
    "0.1B": (12, 768),
    "0.4B": (24, 1024),
    "1.5B": (24, 2048),
    "2.9B": (32, 2560),
    "7.2B": (32, 4096),
    "13.3B": (61, 4096),
}
VOCAB = 65536


def layer_shapes(c):
    """[(matrix id, N, K)] for the six quantized projections of a width-C layer."""
    return [(MAT_R, c, c), (MAT_K, c, c), (MAT_V, c, c), (MAT_O, c, c),
            (MAT_KEY, 4 * c, c), (MAT_VALUE, c, 4 * c)]


def rng(*key):
    """Independent PCG64 stream for a tuple of non-negative ints."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def normal_weight(n, k, g):
    """fp32 [n][k] ~ N(0, 1/k) drawn from generator g."""
    return (g.standard_normal((n, k)) * (1.0 / np.sqrt(k))).astype(np.float32)


def normal_act(m, k, g):
    """fp16 [m][k] ~ N(0, 1)."""
    return g.standard_normal((m, k)).astype(np.float16)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------


def fused_rkv_768():
    """C=768 fused R/K/V: Wr, Wk, Wv fp32 [768][768] and x fp16 [1][768].

    One PCG64(0) stream draws Wr, Wk, Wv, then x, in that order.
    """
    g = np.random.Generator(np.random.PCG64(0))
    ws = [normal_weight(768, 768, g) for _ in range(3)]
    x = normal_act(1, 768, g)
    return ws, x


def weight(cfg, layer, mat, n, k):
    """fp32 weight of matrix ``mat`` in ``layer`` of workload ``cfg``."""
    return normal_weight(n, k, rng(0, cfg, layer, mat))


def act_channel_1202(m, k, cfg=1, salt=0):
    """fp16 [m][k] ~ N(0,1) with column 1202 scaled by 50 (1.5B massive channel)."""
    g = rng(1, cfg, m, k, salt)
    x = g.standard_normal((m, k))
    if k > 1202:
        x[:, 1202] *= 50.0
    return x.astype(np.float16)


def massive_channels(k, cfg=2):
    """Channel set {517} + 7 others, drawn once per width from a fixed stream."""
    g = rng(2, cfg, k)
    others = g.choice(np.setdiff1d(np.arange(k), [517]), size=7, replace=False)
    return np.sort(np.concatenate([[517], others])).astype(np.int64)


def act_massive(m, k, cfg=2, salt=0, frac=0.98):
    """fp16 [m][k]: per row, 8 fixed channels hold ``frac`` of the energy.

    The other entries are N(0,1); each of the 8 channels is set to +-a with
    a^2 = frac * E_rest / ((1 - frac) * 8), E_rest the row's energy outside
    them, random signs.  The split is exact before the fp16 cast.
    """
    ch = massive_channels(k, cfg)
    g = rng(3, cfg, m, k, salt)
    x = g.standard_normal((m, k))
    x[:, ch] = 0.0
    e_rest = np.sum(x * x, axis=1)
    a = np.sqrt(frac * e_rest / ((1.0 - frac) * len(ch)))
    signs = np.where(g.random((m, len(ch))) < 0.5, -1.0, 1.0)
    x[:, ch] = signs * a[:, None]
    return x.astype(np.float16)


def act_normal(m, k, cfg, salt=0):
    """fp16 [m][k] ~ N(0,1) from the stream (4, cfg, m, k, salt)."""
    return normal_act(m, k, rng(4, cfg, m, k, salt))
