"""Per-tensor format maps of the two rwkv-quant presets.

The rwkv-quant news article ("rwkv-quant: uma matriz em bf16 elimina 39% das
perdas na quantização do RWKV-7 2.9B", section "Dois presets e seis tamanhos")
names two presets:

* REDUCTION: projections at 8 bits, symmetric, groups of 16 weights; the
  channel-mix (FFN) matrices at 6 bits; head (and embedding) at 8 bits.
* COMPRESSION: projections at 4 bits in asymmetric superblocks with groups of
  32; the channel-mix at 4 bits except its key matrix at 5 bits; head at
  5 bits (embedding at 6).

Section "Onde o 2.9B quebra" adds one exception: keep the output projection of
the first block in bf16.

The article gives widths, not every layout.  Readings used here:
* 6- and 5-bit weights are the symmetric group formats RQ_W6_SYM / RQ_W5_SYM
  with groups of 32 (the only other group the article states).
* The 4-bit channel-mix value matrix of COMPRESSION uses that preset's 4-bit
  layout, the asymmetric superblocks.
* The 8-bit head of REDUCTION uses the projections' rule (symmetric, group 16).
* The embedding is a row lookup, not a matrix product, and the LoRA branches'
  sizes are not given, so neither is in these maps.

Tensor classes: "r", "k", "v", "o" (time-mix projections), "cmix_key",
"cmix_value" (channel mix), "head".  Each maps to (format, group) with the
format numbers of include/rq.h.
"""

from . import rq

TENSORS = ("r", "k", "v", "o", "cmix_key", "cmix_value", "head")

REDUCTION = {
    "r": (rq.RQ_W8_SYM, 16), "k": (rq.RQ_W8_SYM, 16), "v": (rq.RQ_W8_SYM, 16), "o": (rq.RQ_W8_SYM, 16),
    "cmix_key": (rq.RQ_W6_SYM, 32), "cmix_value": (rq.RQ_W6_SYM, 32),
    "head": (rq.RQ_W8_SYM, 16),
}

COMPRESSION = {
    "r": (rq.RQ_W4_ASYM_SB256, 32), "k": (rq.RQ_W4_ASYM_SB256, 32), "v": (rq.RQ_W4_ASYM_SB256, 32),
    "o": (rq.RQ_W4_ASYM_SB256, 32),
    "cmix_key": (rq.RQ_W5_SYM, 32), "cmix_value": (rq.RQ_W4_ASYM_SB256, 32),
    "head": (rq.RQ_W5_SYM, 32),
}

PRESETS = {"REDUCTION": REDUCTION, "COMPRESSION": COMPRESSION}

# the first block's output projection in bf16 (section "Onde o 2.9B quebra")
BF16_FIRST_O = (rq.RQ_BF16, 0)


def scheme(preset, tensor, layer, bf16_first_o=False):
    """(format, group) of ``tensor`` in ``layer`` under ``preset`` (a name in
    PRESETS); with ``bf16_first_o`` the layer-0 output projection is bf16."""
    if bf16_first_o and tensor == "o" and layer == 0:
        return BF16_FIRST_O
    return PRESETS[preset][tensor]
