"""CPU tests of the small-M launch planner through rq_plan_small_m (host code,
no GPU): for every weight format over ragged and model shapes, m = 1..32,
with and without a workspace, the plan the products would launch must be
well formed (threads, LDS, slices that cover K exactly, workspace within
the caller's bytes, no split without a workspace), deterministic, and
where the planner's choices are documented they are pinned."""

import itertools

import pytest

import gemm_rwkv_amd.rq as rq

LDS_MAX = 160 * 1024
WS = 64 << 20

# (format, group, chunk k)
FORMATS = [(rq.RQ_W4_SYM, 64, 128), (rq.RQ_W4_SYM, 32, 128), (rq.RQ_W4_SYM, 16, 128),
           (rq.RQ_W8_SYM, 64, 64), (rq.RQ_W8_SYM, 32, 64), (rq.RQ_W8_SYM, 16, 64),
           (rq.RQ_W4_ASYM_SB256, 32, 128), (rq.RQ_F16, 0, 32), (rq.RQ_BF16, 0, 32),
           (rq.RQ_W6_SYM, 32, 128), (rq.RQ_W6_SYM, 64, 128), (rq.RQ_W5_SYM, 64, 128)]
NS = [8, 9, 136, 1000, 2048, 2085, 2560, 4072, 4096, 8192, 16384]
KS = [256, 1536, 2048, 2560, 4096, 5120, 5248, 8192, 10240, 16384]
MS = [1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 25, 32]


def _valid_k(fmt, group, k):
    if fmt == rq.RQ_W4_ASYM_SB256:
        return k % 256 == 0
    return k % max(group, 16) == 0


def _plan(fmt, group, n, k, m, ws):
    try:
        return rq.rq_plan_small_m((fmt, group, n, k), m, ws_bytes=ws)
    except rq.RqError as e:
        assert e.status == rq.RQ_ERR_SHAPE, e
        return None


COUNTERS = 64 << 10  # the workspace's leading split counters


@pytest.mark.parametrize("fmt,group,ck", FORMATS)
def test_plans_are_well_formed(fmt, group, ck):
    for n, k, m, ws in itertools.product(NS, KS, MS, (0, WS)):
        if not _valid_k(fmt, group, k):
            continue
        p = _plan(fmt, group, n, k, m, ws)
        where = (fmt, group, n, k, m, ws)
        if p is None:
            # only the formats with a single kernel may find no launch shape
            assert fmt in (rq.RQ_W6_SYM, rq.RQ_W5_SYM, rq.RQ_BF16), where
            continue
        assert p == _plan(fmt, group, n, k, m, ws), where
        assert p["kernel"] in range(1, 6), where
        assert 64 <= p["threads"] <= 1024 and p["threads"] % 64 == 0, where
        assert 0 <= p["lds_bytes"] <= LDS_MAX, where
        assert p["workgroups"] >= 1 and p["split"] >= 1, where
        if p["split"] > 1:
            # the split counters (64 KiB) and then the partial tiles
            assert ws > 0 and COUNTERS < p["workspace_bytes"] <= ws, where
        else:
            assert p["workspace_bytes"] == 0, where
        tiles16 = (n + 15) // 16
        nchunks = k // ck
        if p["kernel"] == rq.RQ_PLAN_FIRST:
            assert p["workgroups"] == tiles16 and p["split"] == 1, where
            continue
        cps, split, rt = p["chunks_per_slice"], p["split"], p["tiles_per_workgroup"]
        # the slices cover K exactly, none empty
        assert (split - 1) * cps < nchunks <= split * cps, where
        if p["kernel"] == rq.RQ_PLAN_PHASED:
            # past 16 rows, or from 9 where it keeps a split in its launch
            assert fmt == rq.RQ_W4_SYM and group in (32, 64) and cps % 4 == 0, where
            assert m > 16 or (m >= 9 and split <= 4), where
            assert p["workgroups"] == -(-tiles16 // rt) * split, where
            # eight waves on two row tiles, sixteen on four
            assert (rt, p["threads"]) in ((2, 512), (4, 1024)), where
            continue
        assert p["waves_per_tile"] * rt * 64 == p["threads"], where
        if p["kernel"] == rq.RQ_PLAN_STREAMED_X and m > 16:
            # the kernel declares at most 512 threads for two activation tiles
            assert p["threads"] <= 512 and rt == 1, where
        span = cps // 2 if p["kernel"] == rq.RQ_PLAN_TWO_RANGES else cps
        assert p["chunks_per_wave"] * p["waves_per_tile"] >= span, where
        assert (p["chunks_per_wave"] * (p["waves_per_tile"] - 1)) < span, where
        if p["kernel"] == rq.RQ_PLAN_TWO_RANGES:
            assert fmt == rq.RQ_W4_SYM and group in (32, 64) and m <= 8 and tiles16 < 256, where
            assert split == 1 and nchunks % 8 == 0 and p["workgroups"] == -(-n // 8), where
        else:
            assert p["workgroups"] == -(-tiles16 // rt) * split, where
        if p["kernel"] == rq.RQ_PLAN_STREAMED_X:
            assert ck == 128 and split == 1 and rt == 1, where
        if fmt == rq.RQ_W4_ASYM_SB256 or (fmt == rq.RQ_W8_SYM and group == 64):
            # superblocks pair chunks; int8 group 64 spans start on whole dwords
            assert cps % 2 == 0 or split == 1, where


def test_documented_plans():
    W4 = (rq.RQ_W4_SYM, 64)
    # width-2048 cmix value: two k ranges at M <= 8, phased in 8 slices at
    # M = 32, the first kernel at M = 32 without a workspace
    p = rq.rq_plan_small_m(W4 + (2048, 8192), 1)
    assert (p["kernel"], p["workgroups"], p["split"]) == (rq.RQ_PLAN_TWO_RANGES, 256, 1)
    p = rq.rq_plan_small_m(W4 + (2048, 8192), 8)
    assert (p["kernel"], p["workgroups"]) == (rq.RQ_PLAN_TWO_RANGES, 256)
    p = rq.rq_plan_small_m(W4 + (2048, 8192), 32)
    # phased, two row tiles per workgroup in four slices summed in the launch
    assert (p["kernel"], p["split"], p["tiles_per_workgroup"], p["workgroups"]) == (rq.RQ_PLAN_PHASED, 4, 2, 256)
    assert p["threads"] == 512
    assert rq.rq_plan_small_m(W4 + (2048, 8192), 32, ws_bytes=0)["kernel"] == rq.RQ_PLAN_FIRST
    # width-4096 cmix value at M = 32: phased, four row tiles on sixteen waves
    p = rq.rq_plan_small_m(W4 + (4096, 16384), 32)
    assert (p["kernel"], p["split"], p["tiles_per_workgroup"], p["threads"]) == (rq.RQ_PLAN_PHASED, 4, 4, 1024)
    # width-4096 cmix key at M = 9..17: phased unsplit on four row tiles,
    # though its activation slice would fit one workgroup whole; the
    # width-2048 K = 2048 shapes, which would need a K split, stay streaming
    for m in (9, 16, 17):
        p = rq.rq_plan_small_m(W4 + (16384, 4096), m)
        assert (p["kernel"], p["split"], p["tiles_per_workgroup"]) == (rq.RQ_PLAN_PHASED, 1, 4), m
        for n in (6144, 8192):
            assert rq.rq_plan_small_m(W4 + (n, 2048), m)["kernel"] == rq.RQ_PLAN_STREAMING, (n, m)
    # width-2048 O (16 chunks) keeps one range
    assert rq.rq_plan_small_m(W4 + (2048, 2048), 1)["kernel"] == rq.RQ_PLAN_STREAMING
    # width-4096 cmix value at M = 1: sixteen-chunk waves, one workgroup of
    # eight waves per row tile; M = 4: K in four slices added in the launch,
    # or, with no workspace, each wave streams its activations
    p = rq.rq_plan_small_m(W4 + (4096, 16384), 1)
    assert (p["kernel"], p["chunks_per_wave"], p["waves_per_tile"], p["workgroups"]) == \
        (rq.RQ_PLAN_STREAMING, 16, 8, 256)
    p = rq.rq_plan_small_m(W4 + (4096, 16384), 4)
    assert (p["kernel"], p["split"]) == (rq.RQ_PLAN_STREAMING, 4)
    assert rq.rq_plan_small_m(W4 + (4096, 16384), 4, ws_bytes=0)["kernel"] == rq.RQ_PLAN_STREAMED_X
    # M > 16: O 4096x4096 streams its activations; SB256 splits instead
    assert rq.rq_plan_small_m(W4 + (4096, 4096), 32)["kernel"] == rq.RQ_PLAN_STREAMED_X
    assert rq.rq_plan_small_m((rq.RQ_W4_ASYM_SB256, 32, 4096, 8192), 32)["kernel"] == rq.RQ_PLAN_STREAMING
    # K is not split at M = 1 for the width-4096 matrices
    for n, k in ((4096, 4096), (16384, 4096), (4096, 16384)):
        assert rq.rq_plan_small_m(W4 + (n, k), 1)["split"] == 1
    # SB256 value matrix at width 2560, M = 1: four slices of waves of four chunks
    p = rq.rq_plan_small_m((rq.RQ_W4_ASYM_SB256, 32, 2560, 10240), 1)
    assert (p["kernel"], p["split"], p["chunks_per_wave"]) == (rq.RQ_PLAN_STREAMING, 4, 4)
    # int4 group 16: the first kernel
    assert rq.rq_plan_small_m((rq.RQ_W4_SYM, 16, 2048, 2048), 1)["kernel"] == rq.RQ_PLAN_FIRST
    # 6-bit, 41 chunks cut 8 ways: 7 non-empty slices of 6
    p = rq.rq_plan_small_m((rq.RQ_W6_SYM, 32, 2085, 5248), 32)
    assert (p["split"], p["chunks_per_slice"]) == (7, 6)


def test_plan_validation():
    d = (rq.RQ_W4_SYM, 64, 2048, 2048)
    assert rq.rq_plan_small_m(d, 0)["kernel"] == rq.RQ_PLAN_NONE
    assert rq.rq_plan_small_m((rq.RQ_W4_SYM, 64, 0, 2048), 4)["kernel"] == rq.RQ_PLAN_NONE
    for bad_m in (-1, 33):
        with pytest.raises(rq.RqError) as e:
            rq.rq_plan_small_m(d, bad_m)
        assert e.value.status == rq.RQ_ERR_SHAPE
    with pytest.raises(rq.RqError) as e:
        rq.rq_plan_small_m(d, 1, ldx=2044)
    assert e.value.status == rq.RQ_ERR_SHAPE
    with pytest.raises(rq.RqError) as e:
        rq.rq_plan_small_m(d, 1, ldx=2052)
    assert e.value.status == rq.RQ_ERR_ALIGN
    with pytest.raises(rq.RqError) as e:
        rq.rq_plan_small_m((rq.RQ_FP8_E4M3_CH, 0, 2048, 2048), 1)
    assert e.value.status == rq.RQ_ERR_FORMAT
    assert rq.lib().rq_plan_small_m(None, 1, 2048, 0, None) == rq.RQ_ERR_NULL


def test_workspace_without_room_past_the_counters_is_none():
    """A workspace of 64 KiB or less holds only the split counters: every
    product plans as with no workspace at all; one byte more admits a split
    only where the partial tiles fit after the counters."""
    for fmt, group, n, k, m in [(rq.RQ_W4_SYM, 64, 2048, 8192, 32), (rq.RQ_W4_SYM, 64, 4096, 16384, 16),
                                (rq.RQ_W4_ASYM_SB256, 32, 2560, 10240, 1), (rq.RQ_W8_SYM, 16, 2560, 10240, 4)]:
        none = _plan(fmt, group, n, k, m, 0)
        full = _plan(fmt, group, n, k, m, WS)
        assert full["split"] > 1, (fmt, n, k, m)
        for ws in (1024, COUNTERS - 16, COUNTERS):
            assert _plan(fmt, group, n, k, m, ws) == none, (fmt, n, k, m, ws)
        assert _plan(fmt, group, n, k, m, full["workspace_bytes"]) == full, (fmt, n, k, m)
        tight = _plan(fmt, group, n, k, m, full["workspace_bytes"] - 16)
        assert tight["split"] == 1 or tight["workspace_bytes"] <= full["workspace_bytes"] - 16
