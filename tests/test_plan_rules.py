"""The dispatch rules, checked on the host through the plan queries (no device).

wq_query_gemm_plan and wq_query_w8a8_plan return the plan a call would take on
a device with a given number of compute units.  These tests pin the plans the
library takes for the FFN and attention shapes on MI355X (256 CUs), which were
chosen from timed sweeps, and check the properties the automatic rules promise
for any shape and CU count: every K group and K part keeps work, parts are only
used with a workspace, and a forced lever is honoured.
"""
import random

import pytest

wq = pytest.importorskip("weight_only_quantized_fp8_amd.wq")

FP8, LUT, LUTD = wq.WQ_FMT_FP8_BLOCK, wq.WQ_FMT_LUT3, wq.WQ_FMT_LUT3_DENSE
GEMV, MFMA = wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA
CU = 256


@pytest.fixture
def levers_reset():
    yield
    wq.wq_set_tuning()
    wq.wq_set_kparts(0)


def plan(fmt, M, N, K, cu=CU, ws=False, path=wq.WQ_PATH_AUTO):
    p = wq.wq_query_gemm_plan(fmt, M, N, K, cu, ws, path)
    return p["nt"], p["sn"], p["split"], p["kparts"]


# (format, N, K): (nt, sn, waves, K parts) without and with a workspace, on 256 CUs
DECODE_PLANS = {
    (FP8, 17408, 5120): ((1, 5, 5, 1), (1, 5, 5, 1)),      # FFN gate/up
    (FP8, 5120, 17408): ((1, 2, 6, 1), (1, 5, 5, 4)),      # FFN down: 4 K parts + the parts sum
    (FP8, 6144, 5120): ((1, 2, 6, 1), (1, 2, 6, 1)),       # attention Q
    (FP8, 1024, 5120): ((1, 1, 4, 1), (1, 1, 4, 1)),       # attention K, V
    (FP8, 8192, 5120): ((1, 2, 6, 1), (1, 2, 6, 1)),       # attention Q, K, V stacked
    (FP8, 5120, 6144): ((1, 2, 6, 1), (1, 2, 6, 1)),       # attention output
    (LUT, 28672, 8192): ((1, 7, 14, 1), (1, 7, 14, 1)),    # 3-bit LUT, nibbles: two K groups
    (LUTD, 28672, 8192): ((1, 8, 16, 1), (1, 8, 16, 1)),   # 3-bit LUT, dense codes: two K groups
}


@pytest.mark.parametrize("key", list(DECODE_PLANS))
def test_measured_decode_plans(key):
    fmt, N, K = key
    no_ws, with_ws = DECODE_PLANS[key]
    for M in (1, 8, 16, 17, 32):
        assert plan(fmt, M, N, K) == no_ws
        assert plan(fmt, M, N, K, ws=True) == with_ws
        p = wq.wq_query_gemm_plan(fmt, M, N, K, CU, True)
        assert p["path"] == MFMA
        assert p["launches"] == 1     # M = 17..32 in one pass on every one-tile table plan


def test_table_applies_only_at_256_cus():
    """The measured plans are for 256 CUs; another count takes the general rule
    (one tile a wave, as many column-waves as leave a work-group per CU)."""
    assert plan(FP8, 16, 17408, 5120, cu=255)[:2] == (1, 4)
    assert plan(FP8, 16, 17408, 5120, cu=304)[:2] == (1, 3)
    assert plan(FP8, 16, 17408, 5120, cu=128)[:2] == (1, 8)
    assert plan(FP8, 16, 5120, 17408, cu=255, ws=True)[3] == 1     # 320 work-groups: no room for parts


def test_gemv_only_when_asked():
    """AUTO never takes the GEMV (the tile ties or wins at every M); an explicit
    GEMV path runs for M <= 4 and is refused above, and for the LUT formats."""
    for M in (1, 2, 4):
        assert wq.wq_query_gemm_plan(FP8, M, 6144, 5120, CU)["path"] == MFMA
        p = wq.wq_query_gemm_plan(FP8, M, 6144, 5120, CU, False, GEMV)
        assert p["path"] == GEMV and (p["nt"], p["sn"], p["split"], p["kparts"]) == (1, 2, 8, 1)
        # a GEMV plan with a workspace keeps K inside the work-group
        assert wq.wq_query_gemm_plan(FP8, M, 5120, 17408, CU, True, GEMV)["kparts"] == 1
    with pytest.raises(wq.WqError) as e:
        wq.wq_query_gemm_plan(FP8, 5, 6144, 5120, CU, False, GEMV)
    assert e.value.status == 9
    with pytest.raises(wq.WqError):
        wq.wq_query_gemm_plan(LUT, 1, 28672, 8192, CU, False, GEMV)


def test_launch_count_follows_the_tile(levers_reset):
    """Rows are served 32 per launch by one-tile waves (FP8 always; LUT where
    its 32-row activation chunks fit), else 16."""
    wq.wq_set_tuning(1, 1, 0, 0)
    assert wq.wq_query_gemm_plan(FP8, 32, 17408, 5120, CU)["launches"] == 1
    assert wq.wq_query_gemm_plan(LUT, 17, 28672, 8192, CU)["launches"] == 2
    assert wq.wq_query_gemm_plan(LUT, 16, 28672, 8192, CU)["launches"] == 1
    wq.wq_set_tuning(1, 4, 0, 0)
    assert wq.wq_query_gemm_plan(LUT, 32, 28672, 8192, CU)["launches"] == 1
    wq.wq_set_tuning(2, 2, 0, 0)
    for fmt, N, K in ((FP8, 17408, 5120), (LUT, 28672, 8192), (LUTD, 28672, 8192)):
        assert wq.wq_query_gemm_plan(fmt, 17, N, K, CU)["launches"] == 2
        assert wq.wq_query_gemm_plan(fmt, 16, N, K, CU)["launches"] == 1


def test_levers_override_the_table(levers_reset):
    wq.wq_set_tuning(1, 4, 8, 0)
    assert plan(FP8, 16, 17408, 5120) == (1, 4, 8, 1)
    assert plan(FP8, 16, 5120, 17408, ws=True)[:3] == (1, 4, 8)
    wq.wq_set_tuning()
    wq.wq_set_kparts(3)
    assert plan(FP8, 16, 17408, 5120, ws=True)[3] == 3
    assert plan(FP8, 16, 17408, 5120)[3] == 1              # parts need a workspace
    wq.wq_set_kparts(32)
    assert plan(FP8, 16, 256, 512, ws=True)[3] == 4        # at most one part per K block
    assert plan(LUT, 16, 48, 1024, ws=True)[3] == 1        # LUT parts keep 8 K blocks


def test_automatic_split_for_low_n_long_k():
    """With a workspace, a grid of at most half the CUs and a long K splits K
    into parts of 32 K blocks or more, to about one work-group per CU."""
    assert plan(FP8, 16, 1024, 16384, ws=True) == (1, 1, 4, 4)
    assert plan(FP8, 16, 1024, 16384) == (1, 1, 4, 1)
    assert plan(FP8, 16, 1024, 16384, cu=128, ws=True)[3] == 2
    assert plan(FP8, 16, 1024, 4096, ws=True)[3] == 1     # 32 K blocks: too short to split


def _general_cases(n=400, seed=7):
    rng = random.Random(seed)
    for _ in range(n):
        fmt = rng.choice((FP8, LUT, LUTD))
        N = rng.choice((128, 256, 384, 1024, 2048, 5120, 8192, 17408, 28672))
        if fmt != FP8:
            N = rng.choice((16, 48, N))
        K = 128 * rng.choice((1, 2, 3, 5, 8, 16, 40, 64, 136, 200))
        cu = rng.choice((1, 8, 80, 104, 128, 228, 255, 256, 304, 1024))
        yield fmt, rng.randint(1, 32), N, K, cu, rng.random() < 0.5


def test_general_rule_invariants():
    """For any shape and CU count: the kernels' limits hold, every K group and
    K part gets at least one (aligned) K block, parts only with a workspace and
    only where they leave about one work-group per CU with 32 K blocks each."""
    for fmt, M, N, K, cu, ws in _general_cases():
        p = wq.wq_query_gemm_plan(fmt, M, N, K, cu, ws)
        nt, sn, split, kp = p["nt"], p["sn"], p["split"], p["kparts"]
        where = (fmt, M, N, K, cu, ws, p)
        kb = K // 128
        align = 8 if fmt != FP8 else 1
        kba = -(-kb // align)
        assert p["path"] == MFMA, where
        assert nt in (1, 2) and 1 <= sn <= 8, where
        assert split % sn == 0 and 1 <= split // sn <= 4 and split <= 16, where
        assert 1 <= kp <= 32 and (split // sn) * kp <= kba, where
        assert p["launches"] in (-(-M // 32), -(-M // 16)), where
        if not ws:
            assert kp == 1, where
        n_cg = -(-(N // 16) // (nt * sn))
        if kp > 1 and cu != 256:
            assert 2 * n_cg <= cu and n_cg * kp <= cu and kb // kp >= 32, where


def test_query_validation():
    assert wq.lib.wq_query_gemm_plan(FP8, 0, 16, 256, 512, CU, 0, None) == 1           # NULL plan
    assert wq.lib.wq_query_w8a8_plan(16, 256, 512, CU, 0, None) == 1
    for args in ((FP8, 0, 256, 512, CU), (FP8, 33, 256, 512, CU), (FP8, 16, 100, 512, CU),
                 (FP8, 16, 256, 500, CU), (LUT, 16, 40, 512, CU), (FP8, 16, 256, 512, 0),
                 (FP8, 16, 256, 512, 1025), (7, 16, 256, 512, CU)):
        with pytest.raises(wq.WqError) as e:
            wq.wq_query_gemm_plan(*args)
        assert e.value.status == 2, args
    with pytest.raises(wq.WqError) as e:
        wq.wq_query_gemm_plan(FP8, 16, 256, 512, CU, False, 3)
    assert e.value.status == 9
    for args in ((0, 256, 512, CU), (16, 100, 512, CU), (16, 256, 500, CU), (16, 256, 512, 0),
                 (16, 65536, 65536, CU), (1 << 25, 256, 512, CU)):
        with pytest.raises(wq.WqError) as e:
            wq.wq_query_w8a8_plan(*args)
        assert e.value.status == 2, args


# W8A8 on 256 CUs, FFN gate/up (17408 x 5120) and down (5120 x 17408):
# M -> (tile rows, tile columns, K parts) with a workspace, and the tile rows
# without one (K whole) -- the choices of the timed sweeps: up to 64 rows the
# weight-streaming tile with the FP8 decode tile's plan (16 / 32 / 64 rows,
# 5 column-waves of 16 columns; down in 4 K parts, or 2 column-waves and K
# whole without a workspace); 128 x 128 split while the grid is short; one
# part for gate/up from M = 192 on; 256 x 256 where its coarser rounds still
# come out ahead (gate/up M = 512, down M = 1024 and 2048 in 3 parts) and
# above M = 4096.  Gate/up M = 1024 / 2048 / 3000 / 4096 and down M = 4096
# run in two column bands (W8A8_BANDS), with or without a workspace: the plan
# listed is that of the leading band.
W8A8_PLANS = {
    "gate_up": {1: ((16, 80, 1), 16), 16: ((16, 80, 1), 16), 32: ((32, 80, 1), 32), 64: ((64, 80, 1), 64),
                96: ((128, 128, 3), 128), 128: ((128, 128, 3), 128), 192: ((128, 128, 1), 128),
                256: ((128, 128, 1), 128), 512: ((256, 256, 1), 256), 1024: ((256, 256, 1), 256),
                2048: ((256, 256, 1), 256), 3000: ((256, 256, 1), 256), 4096: ((256, 256, 1), 256),
                8192: ((256, 256, 1), 256)},
    "down": {1: ((16, 80, 4), 16), 16: ((16, 80, 4), 16), 48: ((64, 80, 4), 64), 64: ((64, 80, 4), 64),
             96: ((128, 128, 6), 128), 128: ((128, 128, 6), 128), 192: ((128, 128, 6), 128),
             256: ((128, 128, 6), 128), 512: ((128, 128, 3), 128), 1024: ((256, 256, 3), 128),
             2048: ((256, 256, 3), 128), 4096: ((256, 256, 1), 256), 8192: ((256, 256, 1), 256)},
}
# (shape, M) -> (columns of the leading band, (tile rows, tile columns, K
# parts) of the rest with a workspace, and without one): the calls whose
# one-band grid would end in a round of work-group slots at most half full
# (gate/up: 1088 128 x 128 tiles on 512 slots at M = 1024, 2176 at 2048; 816
# and 1088 256 x 256 tiles on 256 at M = 3000 and 4096; down M = 4096: 1280
# 128 x 128 tiles on 512), measured 3-17% faster in two bands (2-10%
# without a workspace)
W8A8_BANDS = {("gate_up", 1024): (16384, (128, 128, 3), (128, 128, 1)),
              ("gate_up", 2048): (16384, (128, 128, 2), (128, 128, 1)),
              ("gate_up", 3000): (16384, (256, 256, 3), (128, 128, 1)),
              ("gate_up", 4096): (16384, (256, 256, 3), (128, 128, 1)),
              ("down", 4096): (4096, (256, 256, 3), (128, 128, 1))}
FFN = {"gate_up": (17408, 5120), "down": (5120, 17408)}


@pytest.mark.parametrize("name", list(W8A8_PLANS))
def test_measured_w8a8_plans(name):
    N, K = FFN[name]
    for M, (want, rows_no_ws) in W8A8_PLANS[name].items():
        p = wq.wq_query_w8a8_plan(M, N, K, CU, True)
        assert p["tile"] + (p["kparts"],) == want, (name, M, p)
        assert p["streaming"] == (M <= 64), (name, M, p)
        band, tail, tail_no_ws = W8A8_BANDS.get((name, M), (N, None, None))
        assert (p["band"], p["tail"]) == (band, tail), (name, M, p)
        q = wq.wq_query_w8a8_plan(M, N, K, CU, False)
        assert q["kparts"] == 1 and q["tile"][0] == rows_no_ws, (name, M, q)
        assert (q["band"], q["tail"]) == (band, tail_no_ws), (name, M, q)
    # the streaming tile's columns without a workspace: FFN down's one-part plan (2 column-waves)
    if name == "down":
        assert wq.wq_query_w8a8_plan(16, N, K, CU, False)["tile"] == (16, 32)


def test_w8a8_streaming_only_while_staging_is_small():
    """The streaming tile takes M <= 64 while a work-group's staged activations
    (Mpad x K) are at most twice its weight bytes (16 column-waves x 16 x K):
    attention K/V (one column-wave a work-group) up to 32 rows, then the
    64-row tile kernel."""
    for M in (1, 16, 32):
        assert wq.wq_query_w8a8_plan(M, 1024, 5120, CU, True)["streaming"]
    for M in (33, 48, 64):
        p = wq.wq_query_w8a8_plan(M, 1024, 5120, CU, True)
        assert not p["streaming"] and p["tile"][0] == 64
    for M in (33, 64):
        assert wq.wq_query_w8a8_plan(M, 6144, 5120, CU, True)["streaming"]      # 2 column-waves


def test_w8a8_big_tile_only_where_fitted(levers_reset):
    """The 256 x 256 tile below M = 4097 needs K >= 4096 (the range its cost
    estimate was fitted on) and no forced tile; a forced part count is kept."""
    assert wq.wq_query_w8a8_plan(2049, 2048, 384, CU, False)["tile"] == (128, 128)
    assert wq.wq_query_w8a8_plan(512, 17408, 3968, CU, False)["tile"] == (128, 128)
    assert wq.wq_query_w8a8_plan(512, 17408, 4096, CU, False)["tile"] == (256, 256)
    assert wq.wq_query_w8a8_plan(256, 17408, 5120, CU, False)["tile"] == (128, 128)
    wq.wq_set_kparts(2)
    p = wq.wq_query_w8a8_plan(1024, 5120, 17408, CU, True)
    assert p["kparts"] == 2
    # a forced part count also keeps the call in one band
    p = wq.wq_query_w8a8_plan(4096, 5120, 17408, CU, True)
    assert p["band"] == 5120 and p["tail"] is None


def test_w8a8_forced_parts(levers_reset):
    wq.wq_set_kparts(5)
    assert wq.wq_query_w8a8_plan(16, 5120, 17408, CU, True)["kparts"] == 5
    assert wq.wq_query_w8a8_plan(16, 5120, 17408, CU, False)["kparts"] == 1
    wq.wq_set_kparts(32)
    assert wq.wq_query_w8a8_plan(16, 256, 512, CU, True)["kparts"] == 4


def test_w8a8_rule_invariants():
    """The tile follows the padded row count (256 x 256 below M = 4097 only
    above 256 rows and for K >= 4096); parts keep 12 K blocks or more and
    need a workspace; a split grid of 64-row tiles, or of a 128 x 128 grid
    that fits the CUs, stays within two work-groups per CU; a 128 x 128 grid
    of 1 to 4 tiles per CU adds no part beyond 4 work-groups per CU; a
    256 x 256 grid below M = 4097 splits K (into at most 3) only while it has
    fewer tiles than CUs, and above that keeps K whole."""
    rng = random.Random(11)
    for _ in range(400):
        M = rng.choice((1, 7, 16, 33, 64, 65, 100, 128, 129, 200, 256, 300, 512, 1000, 2048, 4096, 4097, 6000))
        N = 128 * rng.choice((1, 2, 3, 8, 16, 40, 48, 136))
        K = 128 * rng.choice((1, 2, 12, 24, 40, 64, 136))
        cu = rng.choice((8, 80, 128, 256, 304))
        ws = rng.random() < 0.7
        p = wq.wq_query_w8a8_plan(M, N, K, cu, ws)
        (r, c), kp = p["tile"], p["kparts"]
        where = (M, N, K, cu, ws, p)
        mpad = -(-M // 16) * 16
        if p["streaming"]:
            # the weight-streaming tile: the FP8 decode tile's rules (16-row tiles
            # covering Mpad, 1..8 column-waves of 16 columns, parts only with a
            # workspace), staging at most twice a work-group's weight bytes
            assert mpad <= 64 and r == (16 if mpad <= 16 else 32 if mpad <= 32 else 64), where
            assert c % 16 == 0 and 16 <= c <= 128 and mpad <= 2 * c, where
            assert 1 <= kp <= 32 and (ws or kp == 1), where
            continue
        if mpad <= 64:
            assert r == 64, where
        elif mpad > 4096:
            assert r == 256, where
        elif mpad <= 256 or K < 4096:
            assert r == 128, where
        else:
            assert r in (128, 256), where
        assert c == (256 if r == 256 else c) and c in (64, 128, 256), where
        if r != 64:
            assert c == r, where
        nb = p["band"]                                     # the columns of this plan
        tiles = -(-mpad // r) * -(-nb // c)
        if not ws or (r == 256 and (mpad > 4096 or tiles >= cu)):
            assert kp == 1, where
            continue
        if r == 256:
            assert kp <= 3 and K // 128 >= 12 * kp, where
            continue
        if kp > 1:
            assert K // 128 >= 12 * kp or (r == 128 and tiles > cu), where
            if r == 64 or tiles <= cu:
                assert tiles * kp <= 2 * cu, where
            else:
                assert tiles * (kp - 1) < 4 * cu and K // 128 >= 40 * kp, where


def test_w8a8_band_rule_invariants():
    """Two column bands only for 64 < Mpad <= 4096, K >= 4096 and no lever
    set; the leading band is a multiple of 256 columns leaving at most a
    quarter of N, runs in one K part on 128 x 128 or 256 x 256 tiles and fills
    whole rounds of work-group slots (256 x 256 one per CU, 128 x 128 two per
    CU once the grid has more work-groups than CUs); the rest runs on the plan
    of a call over those columns alone, in one K part without a workspace."""
    rng = random.Random(12)
    seen = 0
    for _ in range(600):
        M = rng.choice((65, 129, 300, 512, 897, 1000, 1024, 1500, 2048, 2500, 3000, 3841, 4096, 4097, 8192))
        N = 128 * rng.choice((8, 16, 24, 40, 48, 64, 100, 136))
        K = 128 * rng.choice((12, 24, 40, 48, 64, 136))
        cu = rng.choice((80, 128, 256, 304))
        ws = rng.random() < 0.8
        p = wq.wq_query_w8a8_plan(M, N, K, cu, ws)
        where = (M, N, K, cu, ws, p)
        mpad = -(-M // 16) * 16
        if p["tail"] is None:
            assert p["band"] == N, where
            continue
        seen += 1
        (r, c), kp, na = p["tile"], p["kparts"], p["band"]
        assert 64 < mpad <= 4096 and K >= 4096 and not p["streaming"], where
        assert ws or p["tail"][2] == 1, where
        assert na % 256 == 0 and 0 < na < N and 4 * (N - na) <= N, where
        assert kp == 1 and (r, c) in ((128, 128), (256, 256)), where
        n = -(-mpad // r) * (na // c)
        slots = 2 * cu if (r == 128 and n > cu) else cu
        assert n % slots == 0, where
        q = wq.wq_query_w8a8_plan(M, N - na, K, cu, ws)
        assert q["tile"] + (q["kparts"],) == p["tail"] or q["tail"] is not None, where
    assert seen > 20


def test_w8a8_bands_follow_the_levers(levers_reset):
    """A forced part count keeps one band, with or without a workspace; FFN
    down at M = 2048 without a workspace stays in one band (its rest would be
    a whole extra round of 136 K blocks on half the CUs)."""
    assert wq.wq_query_w8a8_plan(2048, 17408, 5120, CU, True)["tail"] is not None
    assert wq.wq_query_w8a8_plan(2048, 17408, 5120, CU, False)["tail"] == (128, 128, 1)
    assert wq.wq_query_w8a8_plan(2048, 5120, 17408, CU, False)["tail"] is None
    wq.wq_set_kparts(1)
    assert wq.wq_query_w8a8_plan(2048, 17408, 5120, CU, True)["tail"] is None
    assert wq.wq_query_w8a8_plan(2048, 17408, 5120, CU, False)["tail"] is None
    wq.wq_set_kparts(0)
    assert wq.wq_query_w8a8_plan(2048, 17408, 5120, CU, True)["tail"] is not None
