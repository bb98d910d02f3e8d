"""The presets' format maps against the widths the rwkv-quant news article
states (section "Dois presets e seis tamanhos"), through the library's own
byte accounting: bits per weight of each tensor class."""

import gemm_rwkv_amd.rq as rq
from gemm_rwkv_amd import presets


def _bits(fmt, group, k=2560):
    return sum(rq.rq_qweight_bytes(fmt, group, 1, k)) * 8 / k


def test_widths_match_the_article():
    code_bits = {rq.RQ_W8_SYM: 8, rq.RQ_W6_SYM: 6, rq.RQ_W5_SYM: 5, rq.RQ_W4_SYM: 4,
                 rq.RQ_W4_ASYM_SB256: 4, rq.RQ_BF16: 16}
    want = {"REDUCTION": {"r": 8, "k": 8, "v": 8, "o": 8, "cmix_key": 6, "cmix_value": 6, "head": 8},
            "COMPRESSION": {"r": 4, "k": 4, "v": 4, "o": 4, "cmix_key": 5, "cmix_value": 4, "head": 5}}
    for name, table in want.items():
        for t, b in table.items():
            fmt, group = presets.scheme(name, t, 3)
            assert code_bits[fmt] == b, (name, t)
            # stored bits per weight: the code width plus scale overhead
            assert b <= _bits(fmt, group) <= b + 1.0, (name, t, _bits(fmt, group))
    # projections: symmetric groups of 16 in REDUCTION, superblocks of 32 in COMPRESSION
    assert presets.scheme("REDUCTION", "o", 0) == (rq.RQ_W8_SYM, 16)
    assert presets.scheme("COMPRESSION", "o", 0) == (rq.RQ_W4_ASYM_SB256, 32)


def test_bf16_first_output_projection_only():
    assert presets.scheme("COMPRESSION", "o", 0, bf16_first_o=True) == (rq.RQ_BF16, 0)
    assert presets.scheme("COMPRESSION", "o", 1, bf16_first_o=True) == presets.COMPRESSION["o"]
    assert presets.scheme("COMPRESSION", "r", 0, bf16_first_o=True) == presets.COMPRESSION["r"]
