"""K split across work-groups (calls that pass a workspace): each K part's
work-group writes FP32 partial sums to the workspace and a second kernel adds
the parts in order and rounds once.

* against the oracle for forced part counts 1..32 (clamped to the K blocks),
  both formats, M from 1 to 32, ragged column groups, every kernel variant;
  the workspace is filled with NaN bytes before each call, so every partial
  the sum reads must have been written by the call;
* the host rules: workspace size per plan, too small / misaligned workspaces
  rejected before any work, NULL keeping the one-part schedule, the FP8 GEMV
  ignoring the workspace;
* determinism, rows independent of M, HIP-graph replays equal to eager calls;
* the FFN down projection's table plan (four K parts) at full size.
"""
import numpy as np
import pytest
import torch

import synth
import gpu_util as U

pytestmark = pytest.mark.gpu

MFMA, GEMV = 2, 1


@pytest.fixture
def reset():
    yield
    wq = U.wqmod()
    wq.wq_set_kparts(0)
    wq.wq_set_tuning(0, 0, 0, 0)


def workspace(fmt, N, K, fill=0xFF):
    """A workspace of the queried size, pre-filled (0xFF bytes are NaN floats)."""
    wq = U.wqmod()
    t = torch.empty(wq.wq_gemm_workspace_bytes(fmt, 16, N, K), dtype=torch.uint8, device=U.DEV)
    t.fill_(fill)
    return t


def expected_bytes(kp, N, K, align):
    kba = (K // 128 + align - 1) // align
    kp = min(kp, kba)
    return kp * 32 * N * 4 if kp > 1 else 0


@pytest.mark.parametrize("kp", [1, 2, 3, 5, 9, 32])
def test_fp8_parts_match_oracle(kp, reset):
    wq = U.wqmod()
    wq.wq_set_kparts(kp)
    U.note("ksplit fp8 kp=%d" % kp)
    for N, K in ((384, 1152), (640, 640), (128, 256)):
        codes, scales = synth.fp8_weights(N, K, 900 + N)
        packed = U.pack_fp8(codes, scales)
        ws = workspace(wq.WQ_FMT_FP8_BLOCK, N, K)
        assert ws.numel() == expected_bytes(kp, N, K, 1)
        for M in (1, 5, 16, 20, 32):
            ws.fill_(0xFF)
            xb = synth.x_bf16(M, K, 950 + M)
            y, _ = U.run_fp8(packed, N, K, xb, path=MFMA, ws=ws)
            r = U.grade_fp8(y, xb, codes, scales, K)
            U.check(r, "N=%d K=%d M=%d" % (N, K, M))


@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
@pytest.mark.parametrize("kp", [2, 3, 8])
def test_lut3_parts_match_oracle(kp, dense, reset):
    wq = U.wqmod()
    wq.wq_set_kparts(kp)
    U.note("ksplit lut3 kp=%d dense=%d" % (kp, dense))
    fmt = wq.WQ_FMT_LUT3_DENSE if dense else wq.WQ_FMT_LUT3
    for N, K in ((272, 3072), (48, 2048), (80, 1152)):
        c, q, g = synth.lut3_weights(N, K, 960 + N)
        packed = U.pack_lut3(c, q, g, dense=dense)
        ws = workspace(fmt, N, K)
        assert ws.numel() == expected_bytes(kp, N, K, 8)   # parts hold whole runs of 8 K blocks
        for M in (1, 7, 16, 24):
            ws.fill_(0xFF)
            xh = synth.x_f16(M, K, 970 + M)
            y, _ = U.run_lut3(packed, N, K, xh, ws=ws, dense=dense)
            r = U.grade_lut3(y, xh, c, q, g, K)
            U.check(r, "N=%d K=%d M=%d" % (N, K, M), "f16")


# every kernel variant with K parts: one- and two-tile waves, 1..8 column-waves,
# one to four K groups inside each part
TUNINGS = [(1, 1, 4), (2, 1, 3), (1, 2, 4), (2, 2, 8), (1, 3, 6), (1, 5, 5), (1, 7, 14), (1, 8, 8), (2, 8, 8)]


@pytest.mark.parametrize("nt,sn,split", TUNINGS, ids=["nt%d-sn%d-s%d" % t for t in TUNINGS])
def test_every_tiling_with_parts(nt, sn, split, reset):
    wq = U.wqmod()
    wq.wq_set_tuning(nt, sn, split, 0)
    wq.wq_set_kparts(3)
    U.note("ksplit tiling nt=%d sn=%d split=%d" % (nt, sn, split))
    N, K = 640, 2560
    codes, scales = synth.fp8_weights(N, K, 980)
    packed = U.pack_fp8(codes, scales)
    ws = workspace(wq.WQ_FMT_FP8_BLOCK, N, K)
    for M in (3, 16, 29):
        xb = synth.x_bf16(M, K, 981 + M)
        y, _ = U.run_fp8(packed, N, K, xb, path=MFMA, ws=ws)
        r = U.grade_fp8(y, xb, codes, scales, K)
        U.check(r, "fp8 M=%d" % M)
    N, K = 272, 3072
    c, q, g = synth.lut3_weights(N, K, 982)
    packed = U.pack_lut3(c, q, g)
    ws = workspace(wq.WQ_FMT_LUT3, N, K)
    for M in (2, 16, 25):
        xh = synth.x_f16(M, K, 983 + M)
        y, _ = U.run_lut3(packed, N, K, xh, ws=ws)
        r = U.grade_lut3(y, xh, c, q, g, K)
        U.check(r, "lut3 M=%d" % M, "f16")


def test_host_rules(reset):
    wq = U.wqmod()
    U.note("ksplit host rules")
    N, K = 384, 1152
    codes, scales = synth.fp8_weights(N, K, 990)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(16, K, 991)
    x = U.t_u16(xb, torch.bfloat16)
    y = torch.empty((16, N), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_set_kparts(4)
    need = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, 16, N, K)
    assert need == 4 * 32 * N * 4
    assert all(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, M, N, K) == need for M in (1, 7, 32))
    big = torch.zeros(need + 64, dtype=torch.uint8, device=U.DEV)
    y.fill_(7.0)
    with pytest.raises(wq.WqError) as e:                          # too small
        wq.wq_gemm_fp8_block_path(packed, N, K, x, y, 16, big[:need - 16], MFMA)
    assert e.value.status == 4
    with pytest.raises(wq.WqError) as e:                          # misaligned
        wq.wq_gemm_fp8_block_path(packed, N, K, x, y, 16, big[4:4 + need], MFMA)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((y.float() == 7.0).all())                        # rejected calls queue nothing
    # NULL keeps the one-part schedule: the same bits as with the hook at 1
    y_null, _ = U.run_fp8(packed, N, K, xb, path=MFMA)
    wq.wq_set_kparts(1)
    assert wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, 16, N, K) == 0
    y_one, _ = U.run_fp8(packed, N, K, xb, path=MFMA, ws=big)
    assert np.array_equal(y_null, y_one)
    # the GEMV keeps its K split inside the work-group: a workspace changes nothing
    wq.wq_set_kparts(4)
    for M in (1, 3):
        a, _ = U.run_fp8(packed, N, K, xb[:M], path=GEMV)
        b, _ = U.run_fp8(packed, N, K, xb[:M], path=GEMV, ws=big[:need])
        assert np.array_equal(a, b), M


def test_determinism_and_rows(reset):
    wq = U.wqmod()
    wq.wq_set_kparts(5)
    U.note("ksplit determinism")
    N, K = 640, 2560
    codes, scales = synth.fp8_weights(N, K, 992)
    packed = U.pack_fp8(codes, scales)
    ws = workspace(wq.WQ_FMT_FP8_BLOCK, N, K)
    x32 = synth.x_bf16(32, K, 993)
    y32, _ = U.run_fp8(packed, N, K, x32, path=MFMA, ws=ws)
    y16, _ = U.run_fp8(packed, N, K, x32[:16], path=MFMA, ws=ws)
    assert np.array_equal(y32[:16], y16)
    for M in (1, 6, 13):
        yM, _ = U.run_fp8(packed, N, K, x32[:M], path=MFMA, ws=ws)
        assert np.array_equal(yM, y16[:M]), M
    for i in range(10):
        ws.fill_(i * 37 % 256)
        yr, _ = U.run_fp8(packed, N, K, x32, path=MFMA, ws=ws)
        assert np.array_equal(yr, y32), i


def test_graph_replay_with_parts(reset):
    """The GEMM and the parts sum captured in a HIP graph replay to the eager result."""
    wq = U.wqmod()
    wq.wq_set_kparts(4)
    U.note("ksplit graph replay")
    N, K, M = 640, 2560, 16
    codes, scales = synth.fp8_weights(N, K, 994)
    packed = U.pack_fp8(codes, scales)
    ws = workspace(wq.WQ_FMT_FP8_BLOCK, N, K)
    x = U.t_u16(synth.x_bf16(M, K, 995), torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_gemm_fp8_block_path(packed, N, K, x, y, M, ws, MFMA)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            wq.wq_gemm_fp8_block_path(packed, N, K, x, y, M, ws, MFMA)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.fill_(3.0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.parametrize("M", [4, 16, 32])
def test_down_projection_table_plan(M, reset):
    """FFN down 5120 x 17408 with a workspace: the table plan splits K in four
    parts (sampled columns against the oracle, as the full-size config tests)."""
    wq = U.wqmod()
    fmt, N, K, Ms, (codes, scales) = U.config_inputs("down")
    assert wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, M, N, K) == 4 * 32 * N * 4
    U.note("ksplit down M=%d" % M)
    packed = U.pack_fp8(codes, scales)
    ws = workspace(wq.WQ_FMT_FP8_BLOCK, N, K)
    xb = synth.x_bf16(M, K, synth.SEEDS["down"] + 200 + M)
    y, _ = U.run_fp8(packed, N, K, xb, path=MFMA, ws=ws)
    cols = U.sample_cols(N, 17 + M)
    r = U.grade_fp8(y, xb, codes, scales, K, cols=cols)
    U.note("  %s" % r)
    U.check(r)


def test_plan_query_matches_the_device():
    """The host plan queries, given this device's CU count, give the K parts
    the calls size their workspaces for (decode GEMMs and W8A8)."""
    wq = U.wqmod()
    U.note("ksplit plan query against the device")
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    for fmt, N, K in ((wq.WQ_FMT_FP8_BLOCK, 17408, 5120), (wq.WQ_FMT_FP8_BLOCK, 5120, 17408),
                      (wq.WQ_FMT_FP8_BLOCK, 1024, 5120), (wq.WQ_FMT_FP8_BLOCK, 1024, 16384),
                      (wq.WQ_FMT_LUT3, 28672, 8192), (wq.WQ_FMT_LUT3_DENSE, 28672, 8192),
                      (wq.WQ_FMT_LUT3, 48, 8192)):
        kp = wq.wq_query_gemm_plan(fmt, 16, N, K, cu, True)["kparts"]
        assert wq.wq_gemm_workspace_bytes(fmt, 16, N, K) == (kp * 32 * N * 4 if kp > 1 else 0), (fmt, N, K, kp)
    for M, N, K in ((16, 17408, 5120), (16, 5120, 17408), (128, 5120, 17408), (1024, 5120, 17408),
                    (8192, 17408, 5120), (300, 1280, 1152), (2048, 17408, 5120), (4096, 5120, 17408)):
        p = wq.wq_query_w8a8_plan(M, N, K, cu, True)
        kp, n = (p["tail"][2], N - p["band"]) if p["tail"] else (p["kparts"], N)
        assert wq.wq_w8a8_workspace_bytes(M, N, K) == (kp * M * n * 4 if kp > 1 else 0), (M, N, K, p)
