"""W8A8 tier on the GPU (called through the C ABI) against the CPU oracle.

* quantiser: the packed FP8 activations, unpacked by the test hook, equal the
  oracle's codes and scales bit for bit (the codes are an integer decision made
  in binary32 on both sides), padding rows are zero;
* GEMM: every output within 2 BF16 ULP of the oracle's exact sum of the
  quantised operands, or within the absolute floor, on shapes with ragged row
  tiles, several column tiles and K blocks, M from 1 to a few hundred and at
  the FFN gate/up size; integer-exact inputs give exact results; rows are
  independent of M, results deterministic, y's padding untouched, HIP-graph
  replays equal the eager result;
* LDS pipeline depth: two and four stages give bitwise equal outputs, and at
  the FFN sizes small-M calls (four stages) equal the first rows of an
  M = 2048 call (two stages);
* K split across work-groups (a workspace passed): forced part counts against
  the oracle (NaN-filled workspace), the automatic split of the FFN down
  projection, workspace errors, determinism and graph replay.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import gpu_util as U
from oracle import compare

pytestmark = pytest.mark.gpu


def quantize(xbits, K):
    """GPU-quantised activations of BF16 bits [M, ldx]: (packed buffer, codes, scales)."""
    wq = U.wqmod()
    M = xbits.shape[0]
    x = U.t_u16(xbits, torch.bfloat16)
    xq = torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=U.DEV)
    xq.fill_(0xA5)                                        # padding must be written, not left over
    wq.wq_quantize_x_fp8(x[:, :K] if xbits.shape[1] > K else x, M, K, xq)
    codes = torch.empty((M, K), dtype=torch.uint8, device=U.DEV)
    scales = torch.empty((M, K // 128), dtype=torch.float32, device=U.DEV)
    wq.wq_unpack_x_fp8(xq, M, K, codes, scales)
    torch.cuda.synchronize()
    return xq, codes.cpu().numpy(), scales.cpu().numpy()


def run(packed, N, K, xq, M, ldy=None, y_init=None, ws=None):
    """ws: None (no workspace), "auto" (wq_w8a8_workspace_bytes, NaN-filled) or a buffer."""
    wq = U.wqmod()
    ldy = N if ldy is None else ldy
    y = torch.empty((M, ldy), dtype=torch.bfloat16, device=U.DEV)
    if y_init is not None:
        y.copy_(U.t_u16(y_init, torch.bfloat16))
    if isinstance(ws, str):
        nb = wq.wq_w8a8_workspace_bytes(M, N, K)
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=U.DEV) if nb else None
    wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, ws)
    torch.cuda.synchronize()
    full = U.bits_of(y)
    return full[:, :N], full


# Outputs beyond 2 BF16 ULP (all inside the floor) that the FP8 x FP8 tier may
# show: its matrix core sums a K block's 128 FP8 products less exactly than
# FP32 round-to-nearest, so small outputs (cancellations) miss the ULP budget
# more often than on the decode paths -- measured 6e-4 .. 8e-4 of the outputs
# at M = 16 .. 1030 and 1 of 256 at M = 1, with rel_rms at the BF16 rounding
# level (1.6e-3) and integer-exact inputs exact.
W8A8_OVER_FRAC = 2e-3


def check_w8a8(r):
    U.check(r, "w8a8", max_over=max(1, int(W8A8_OVER_FRAC * r.n)))


def floor_w8a8(xc, xs, codes, scales, K):
    mx = float(np.abs(oracle.e4m3_value(xc) * np.repeat(xs.astype(np.float64), 128, 1)).max())
    mw = 0.0
    for r0 in range(0, codes.shape[0], 2048):
        w = oracle.dequant_fp8(codes[r0:r0 + 2048], scales[r0 // 128:(r0 + 2048) // 128])
        mw = max(mw, float(np.abs(w).max()))
    return compare.abs_floor(K, mx, mw)


def special_x(M, K, seed, ld=None):
    """BF16 activations with an all-zero group, a group holding 448 (scale 1), a
    negative extreme, tiny and huge groups, and NaN canaries in any padding."""
    x = synth.normal_matrix(M, K, seed)
    if M > 3 and K >= 256:
        x[1, 128:256] = 0.0
        x[2, 0:128] = np.abs(x[2, 0:128])
        x[2, 5] = -11.0
        x[3, 0:128] = np.clip(x[3, 0:128] * 50, -447, 447)
        x[3, 17] = 448.0
        x[0, 0:128] *= 1e-5
        x[0, 128:256] *= 2e4
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if ld is not None and ld > K:
        wide = np.full((M, ld), 0x7FC1, dtype=np.uint16)
        wide[:, :K] = bits
        return wide
    return bits


@pytest.mark.parametrize("M,K,ld", [(1, 128, None), (5, 512, None), (16, 384, 392), (37, 1024, None),
                                    (300, 640, 648)])
def test_quantizer_matches_oracle_bit_exact(M, K, ld):
    U.note("w8a8 quantize M=%d K=%d ld=%s" % (M, K, ld))
    xb = special_x(M, K, 60 + M, ld)
    xq, codes, scales = quantize(xb, K)
    oc, osc = oracle.quantize_x_fp8(xb, K=K)
    assert np.array_equal(scales.view(np.uint32), osc.view(np.uint32)), "scales differ"
    assert np.array_equal(codes, oc), "codes differ at %s" % (np.argwhere(codes != oc)[:4],)
    # padding rows: zero codes and zero scales
    wq = U.wqmod()
    Mpad = (M + 15) // 16 * 16
    raw = xq.cpu().numpy()
    assert raw.size == wq.wq_x_fp8_packed_bytes(M, K) == Mpad * K + 4 * Mpad * (K // 128)
    sx = raw[Mpad * K:].view(np.float32).reshape(K // 128, Mpad)
    assert not sx[:, M:].any()
    if Mpad > M:
        units = raw[:Mpad * K].reshape(Mpad // 16, K // 128, 2, 64, 16)
        last = units[-1]                                  # rows 16*(tiles-1) .. Mpad-1
        lanes = np.arange(64) % 16 + 16 * (Mpad // 16 - 1) >= M
        assert not last[:, :, lanes, :].any()


def test_quantizer_every_bf16_magnitude():
    """Every finite BF16 value x (both signs, zeros and subnormals included)
    with |x| <= amax, for amax across the binades -- from the smallest BF16
    subnormal, through both sides of 2^-80 (below which the quantiser divides
    by the scale, above which it multiplies by its correctly rounded
    reciprocal and corrects the remainder), to the largest finite BF16 -- in
    groups whose amax it is (the group's first value): codes and scales equal
    the oracle's bit for bit (the oracle divides)."""
    allx = np.arange(65536, dtype=np.uint32)
    xs = allx[(allx & 0x7F80) != 0x7F80].astype(np.uint16)   # finite patterns
    mag = xs & 0x7FFF                                           # BF16 magnitude order = integer order
    amaxes = [0x0001, 0x0025, 0x0080, 0x0711, 0x0B80, 0x1234, 0x1700, 0x177F, 0x1780, 0x1781, 0x17F3,
              0x1F00, 0x2A55, 0x3381, 0x3C00, 0x3F80, 0x3FC1, 0x4000, 0x43E0, 0x4B2B, 0x55AA, 0x5F12,
              0x6C00, 0x7700, 0x7F7F]
    groups = []
    for a in amaxes:
        sel = xs[mag <= a]
        n = -(-len(sel) // 127)
        g = np.zeros((n, 128), dtype=np.uint16)
        g[:, 0] = a
        flat = np.zeros(n * 127, dtype=np.uint16)
        flat[:len(sel)] = sel
        g[:, 1:] = flat.reshape(n, 127)
        groups.append(g)
    groups = np.concatenate(groups)
    K = 4096
    M = -(-len(groups) // (K // 128))
    xb = np.zeros((M * (K // 128), 128), dtype=np.uint16)
    xb[:len(groups)] = groups
    xb = xb.reshape(M, K)
    U.note("w8a8 quantize every BF16 magnitude: %d groups, M=%d K=%d" % (len(groups), M, K))
    xq, codes, scales = quantize(xb, K)
    oc, osc = oracle.quantize_x_fp8(xb, K=K)
    assert np.array_equal(scales.view(np.uint32), osc.view(np.uint32)), "scales differ"
    bad = np.argwhere(codes != oc)
    assert not len(bad), "codes differ at %s (x %s)" % (bad[:4], [hex(xb[tuple(i)]) for i in bad[:4]])


def test_quantizer_nonfinite_groups():
    """A K group holding +Inf, -Inf or NaN quantises to a NaN scale and the
    E4M3 NaN code everywhere, as in the oracle; every output of its row is NaN
    and every other output passes the oracle."""
    M, N, K = 20, 384, 512
    U.note("w8a8 non-finite activations")
    xb = special_x(M, K, 71)
    xb[0, 5] = 0x7F80
    xb[6, 300] = 0xFF80
    xb[19, 511] = 0x7FC1
    xq, codes, scales = quantize(xb, K)
    oc, osc = oracle.quantize_x_fp8(xb, K=K)
    assert np.array_equal(np.isnan(scales), np.isnan(osc)) and np.isnan(osc).sum() == 3
    fin = ~np.isnan(osc)
    assert np.array_equal(scales[fin].view(np.uint32), osc[fin].view(np.uint32))
    assert np.array_equal(codes, oc)
    wcodes, wscales = synth.fp8_weights(N, K, 72)
    y, _ = run(U.pack_fp8(wcodes, wscales), N, K, xq, M)
    yv = oracle.bf16_value(y)
    bad = [0, 6, 19]
    good = [m for m in range(M) if m not in bad]
    assert np.all(np.isnan(yv[bad])) and np.all(np.isfinite(yv[good]))
    y64 = oracle.gemm_w8a8(oc[good], osc[good], wcodes, wscales)
    check_w8a8(compare.grade(y[good], y64, floor_w8a8(oc[good], osc[good], wcodes, wscales, K), "bf16"))


# M above 4096 runs the 256 x 256 work-group tile (WQ_W8A8_TILE=256 forces it
# for every M; 384 and 640 columns leave a ragged column tile there), smaller M
# the 128 x 128 one
W8A8_SHAPES = [(128, 128, 5), (128, 128, 33), (256, 512, 1), (384, 1024, 16), (1024, 640, 33), (640, 2048, 130),
               (256, 256, 300),
               (512, 1152, 129), (384, 1024, 700), (640, 768, 530), (1280, 512, 1030), (384, 512, 4100),
               (640, 256, 4400)]


@pytest.mark.parametrize("N,K,M", W8A8_SHAPES)
def test_w8a8_parity(N, K, M):
    U.note("w8a8 parity N=%d K=%d M=%d" % (N, K, M))
    codes, scales = synth.fp8_weights(N, K, 1100 + N + K)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 1200 + M)
    xq, xc, xs = quantize(xb, K)
    oc, osc = oracle.quantize_x_fp8(xb)
    assert np.array_equal(xc, oc) and np.array_equal(xs, osc)
    y, _ = run(packed, N, K, xq, M)
    y64 = oracle.gemm_w8a8(oc, osc, codes, scales)
    r = compare.grade(y, y64, floor_w8a8(oc, osc, codes, scales, K), "bf16")
    check_w8a8(r)


def test_w8a8_integer_exact():
    U.note("w8a8 integer exact")
    rng = np.random.Generator(np.random.PCG64(61))
    N, K, M = 256, 1024, 40
    xi = rng.integers(-6, 7, size=(M, K)).astype(np.int64)
    xi[:, ::128] = 448                                    # every group quantises with scale 1
    wi = rng.integers(-8, 9, size=(N, K))
    xb = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = torch.from_numpy(wi.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    packed = U.pack_fp8(q, np.ones((N // 128, K // 128), np.float32))
    xq, _, xs = quantize(xb, K)
    assert np.all(xs == 1.0)
    y, _ = run(packed, N, K, xq, M)
    assert np.array_equal(y, oracle.bf16_rne((xi @ wi.T).astype(np.float64)))


def test_w8a8_rows_determinism_strides():
    """Row r of the result depends only on row r of the activations, for each
    kernel: calls of at most 32 rows (here the weight-streaming tile, whose
    plan does not depend on M) equal the matching rows of a 32-row call, calls
    of more than 64 (the tile kernels, K whole) those of a 150-row call, and the 256 x 256
    tile (M > 4096) folds the same MFMA blocks in the same order as 128 x 128;
    repeats are deterministic and a wider row stride leaves the pad alone."""
    wq = U.wqmod()
    U.note("w8a8 invariants")
    N, K, M = 384, 768, 150
    codes, scales = synth.fp8_weights(N, K, 62)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 63)
    xq, _, _ = quantize(xb, K)
    y, _ = run(packed, N, K, xq, M)
    xq64, _, _ = quantize(xb[:32], K)
    assert wq.wq_query_w8a8_plan(32, N, K, 256, False)["streaming"]
    y64, _ = run(packed, N, K, xq64, 32)
    for lo, hi in ((0, 20), (20, 32), (16, 17)):
        xq2, _, _ = quantize(xb[lo:hi], K)
        y2, _ = run(packed, N, K, xq2, hi - lo)
        assert np.array_equal(y2, y64[lo:hi]), (lo, hi)
    for lo, hi in ((0, 100), (70, 150)):
        xq2, _, _ = quantize(xb[lo:hi], K)
        y2, _ = run(packed, N, K, xq2, hi - lo)
        assert np.array_equal(y2, y[lo:hi]), (lo, hi)
    for _ in range(5):
        assert np.array_equal(run(packed, N, K, xq, M)[0], y)
        assert np.array_equal(run(packed, N, K, xq64, 32)[0], y64)
    xbig = np.vstack([xb, synth.x_bf16(4200 - M, K, 64)])
    xqb, _, _ = quantize(xbig, K)
    yb, _ = run(packed, N, K, xqb, 4200)
    assert np.array_equal(yb[:M], y)
    ldy = N + 40
    for Mc, xqc, ref in ((M, xq, y), (32, xq64, y64)):
        canary = np.full((Mc, ldy), 0x7FAB, dtype=np.uint16)
        ys, full = run(packed, N, K, xqc, Mc, ldy=ldy, y_init=canary)
        assert np.array_equal(ys, ref) and np.all(full[:, N:] == 0x7FAB), Mc


def test_w8a8_graph_replay():
    """Quantiser and GEMM captured in a HIP graph replay to the eager result."""
    wq = U.wqmod()
    U.note("w8a8 graph replay")
    N, K, M = 512, 1024, 96
    codes, scales = synth.fp8_weights(N, K, 64)
    packed = U.pack_fp8(codes, scales)
    x = U.t_u16(synth.x_bf16(M, K, 65), torch.bfloat16)
    xq = torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=U.DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_quantize_x_fp8(x, M, K, xq)
    wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            wq.wq_quantize_x_fp8(x, M, K, xq)
            wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.fill_(3.0)
        xq.fill_(0x11)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.parametrize("M", [64, 512, 1024])
def test_w8a8_gate_up_size(M):
    """The FFN gate/up matrix (17408 x 5120): every column of the first and last
    128 and 768 random ones in between, all M rows."""
    U.note("w8a8 gate_up M=%d" % M)
    fmt, N, K, Ms, (codes, scales) = U.config_inputs("gate_up")
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 1301)
    xq, xc, xs = quantize(xb, K)
    oc, osc = oracle.quantize_x_fp8(xb)
    assert np.array_equal(xc, oc) and np.array_equal(xs, osc)
    y, _ = run(packed, N, K, xq, M)
    cols = U.sample_cols(N, 66)
    y64 = oracle.gemm_w8a8(oc, osc, codes, scales, cols=cols)
    r = compare.grade(y[:, cols], y64, floor_w8a8(oc, osc, codes, scales, K), "bf16")
    U.note("  %s" % r)
    check_w8a8(r)


# ------------------------------------------------------------ pipeline depth

@pytest.fixture
def stages_reset():
    yield
    U.wqmod().wq_set_w8a8_stages(0)
    U.wqmod().wq_set_kparts(0)


@pytest.mark.parametrize("N,K,M,kp", [(256, 512, 1, 0), (384, 1024, 16, 0), (640, 2048, 130, 0),
                                      (1280, 512, 1030, 0), (384, 1024, 700, 3), (640, 2048, 33, 5)])
def test_w8a8_pipeline_depths_agree(N, K, M, kp, stages_reset):
    """Two and four LDS stages run the same arithmetic: bitwise equal outputs
    (with and without K parts), and the automatic choice agrees with both."""
    wq = U.wqmod()
    U.note("w8a8 stages N=%d K=%d M=%d kp=%d" % (N, K, M, kp))
    codes, scales = synth.fp8_weights(N, K, 1600 + N + K)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 1700 + M)
    xq, xc, xs = quantize(xb, K)
    wq.wq_set_kparts(kp)
    out = {}
    for ns in (2, 4, 0):
        wq.wq_set_w8a8_stages(ns)
        out[ns] = run(packed, N, K, xq, M, ws="auto" if kp else None)[0]
    assert np.array_equal(out[2], out[4]) and np.array_equal(out[0], out[2])
    y64 = oracle.gemm_w8a8(xc, xs, codes, scales)
    check_w8a8(compare.grade(out[4], y64, floor_w8a8(xc, xs, codes, scales, K), "bf16"))


@pytest.mark.parametrize("M", [2048, 2049])
def test_w8a8_depth_boundary(M, stages_reset):
    """N = 2048: M = 2048 gives 16 x 16 = 256 work-groups, the most the
    four-stage pipeline takes on a 256-CU part; M = 2049 gives 17 x 16 = 272
    (two stages).  Both against the oracle on sampled columns, and equal to
    the forced other depth."""
    wq = U.wqmod()
    N, K = 2048, 384
    U.note("w8a8 depth boundary N=%d K=%d M=%d" % (N, K, M))
    codes, scales = synth.fp8_weights(N, K, 1900)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 1901)
    xq, xc, xs = quantize(xb, K)
    y, _ = run(packed, N, K, xq, M)
    for ns in (2, 4):
        wq.wq_set_w8a8_stages(ns)
        assert np.array_equal(run(packed, N, K, xq, M)[0], y), ns
    cols = U.sample_cols(N, 68)
    y64 = oracle.gemm_w8a8(xc, xs, codes, scales, cols=cols)
    check_w8a8(compare.grade(y[:, cols], y64, floor_w8a8(xc, xs, codes, scales, K), "bf16"))


@pytest.mark.parametrize("name,small", [("gate_up", (16, 48, 128, 512)), ("down", (128,))])
def test_w8a8_small_grid_rows_equal_large_grid(name, small, stages_reset):
    """At the FFN sizes M = 2048 runs FFN down on 128 x 128 tiles on the
    two-stage pipeline and gate/up in two column bands (256 x 256 tiles, then
    the last 1024 columns on 128 x 128, K whole in both); gate/up M = 16 and
    48 run the weight-streaming tile (one K group, so the same fold order),
    M = 128 the four-stage pipeline (at most one work-group per CU), and
    gate/up M = 512 the 256 x 256 tile.  Rows depend
    only on their own activations, so the smaller calls equal the first rows
    of the large one bit for bit.  (FFN down at M <= 64 without a workspace
    streams with 3 K groups, another summation order: graded against the
    oracle by the parity tests.)"""
    wq = U.wqmod()
    fmt, N, K, Ms, (codes, scales) = U.config_inputs(name)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(2048, K, 1801)
    xq, _, _ = quantize(xb, K)
    U.note("w8a8 %s M=2048 (two stages)" % name)
    p = wq.wq_query_w8a8_plan(2048, N, K, 256, False)
    assert (p["tile"], p["tail"]) == (((256, 256), (128, 128, 1)) if name == "gate_up" else ((128, 128), None))
    ybig, _ = run(packed, N, K, xq, 2048)
    for M in small:
        U.note("w8a8 %s M=%d (plan %s)" % (name, M, wq.wq_query_w8a8_plan(M, N, K, 256, False)))
        xq2, _, _ = quantize(xb[:M], K)
        y, _ = run(packed, N, K, xq2, M)
        assert np.array_equal(y, ybig[:M]), M


# ---------------------------------------------------------- K parts (workspace)

@pytest.fixture
def kparts_reset():
    yield
    U.wqmod().wq_set_kparts(0)


@pytest.mark.parametrize("kp", [2, 3, 7])
@pytest.mark.parametrize("N,K,M", [(384, 1024, 16), (640, 2048, 130), (1280, 1152, 300), (384, 3072, 4100)])
def test_w8a8_parts_match_oracle(N, K, M, kp, kparts_reset):
    wq = U.wqmod()
    wq.wq_set_kparts(kp)
    U.note("w8a8 parts N=%d K=%d M=%d kp=%d" % (N, K, M, kp))
    assert wq.wq_w8a8_workspace_bytes(M, N, K) == min(kp, K // 128) * M * N * 4
    codes, scales = synth.fp8_weights(N, K, 1400 + N + K)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 1500 + M)
    xq, xc, xs = quantize(xb, K)
    y, _ = run(packed, N, K, xq, M, ws="auto")
    y64 = oracle.gemm_w8a8(xc, xs, codes, scales)
    r = compare.grade(y, y64, floor_w8a8(xc, xs, codes, scales, K), "bf16")
    check_w8a8(r)
    for _ in range(3):                                    # deterministic, whatever the workspace held
        assert np.array_equal(run(packed, N, K, xq, M, ws="auto")[0], y)


@pytest.mark.parametrize("name,M,kp", [("down", 256, 6), ("down", 128, 6), ("down", 64, 4), ("gate_up", 64, 1),
                                       ("gate_up", 128, 3), ("down", 1024, 3)])
def test_w8a8_automatic_split(name, M, kp, kparts_reset):
    """The automatic plan at the FFN sizes: FFN down at M = 256 in 6 K parts
    (80 128 x 128 tiles, two work-groups per CU), at M = 128 in 6 (40 tiles),
    at M = 64 on the weight-streaming tile in 4 (the FP8 decode tile's plan),
    at M = 1024 in 3 on 256 x 256 tiles (80 tiles, one work-group per CU);
    gate/up at M = 64 on the streaming tile with K whole, at M = 128 in 3 and
    with K whole from M = 256 on (sampled columns against the oracle)."""
    wq = U.wqmod()
    fmt, N, K, Ms, (codes, scales) = U.config_inputs(name)
    assert wq.wq_w8a8_workspace_bytes(M, N, K) == (kp * M * N * 4 if kp > 1 else 0)
    assert wq.wq_w8a8_workspace_bytes(256, 17408, 5120) == 0        # gate/up keeps K whole
    U.note("w8a8 %s M=%d with a workspace (%d parts)" % (name, M, kp))
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 1601)
    xq, xc, xs = quantize(xb, K)
    y, _ = run(packed, N, K, xq, M, ws="auto")
    cols = U.sample_cols(N, 67)
    y64 = oracle.gemm_w8a8(xc, xs, codes, scales, cols=cols)
    r = compare.grade(y[:, cols], y64, floor_w8a8(xc, xs, codes, scales, K), "bf16")
    U.note("  %s" % r)
    check_w8a8(r)


@pytest.mark.parametrize("N,K,M,kp", [(1408, 4608, 1500, 3), (2432, 4096, 1000, 2), (3200, 4096, 3000, 1)])
def test_w8a8_automatic_big_tile(N, K, M, kp):
    """Ragged shapes (N not a multiple of 256, M not of 16) on which the
    automatic plan takes the 256 x 256 tile below M = 4097, in 3, 2 and 1 K
    parts: sampled columns against the oracle, and the same bits on a repeat
    (NaN-filled workspace)."""
    wq = U.wqmod()
    U.note("w8a8 big tile N=%d K=%d M=%d kp=%d" % (N, K, M, kp))
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if cu == 256:
        p = wq.wq_query_w8a8_plan(M, N, K, cu, True)
        assert (p["tile"], p["kparts"], p["streaming"], p["tail"]) == ((256, 256), kp, False, None)
    codes, scales = synth.fp8_weights(N, K, 2100 + N)
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 2200 + M)
    xq, xc, xs = quantize(xb, K)
    y, _ = run(packed, N, K, xq, M, ws="auto")
    cols = U.sample_cols(N, 69, 160)
    y64 = oracle.gemm_w8a8(xc, xs, codes, scales, cols=cols)
    r = compare.grade(y[:, cols], y64, floor_w8a8(xc, xs, codes, scales, K), "bf16")
    U.note("  %s" % r)
    check_w8a8(r)
    assert np.array_equal(run(packed, N, K, xq, M, ws="auto")[0], y)


@pytest.mark.parametrize("name,M", [("gate_up", 1024), ("gate_up", 2048), ("gate_up", 3000), ("down", 4096),
                                    ((9600, 4096), 1793)])
def test_w8a8_column_bands(name, M):
    """Calls whose one-band grid would end in a mostly idle round of
    work-group slots run in two column bands.  The leading band (one K part)
    equals the call without a workspace (K whole in every tile, also in two
    bands) bit for bit, and that call equals the one-band plan (one K part
    forced); the remaining columns equal a call of their own on those
    columns' packed matrix, whose plan is the band's; sampled columns of both
    bands, and the columns around the band edge, against the oracle
    (NaN-filled workspaces).  The 9600-column shape at M = 1793 has ragged
    rows and ends its second band (1408 columns on 256 x 256 tiles, in 2 K
    parts) with a half-filled tile."""
    wq = U.wqmod()
    if isinstance(name, tuple):
        N, K = name
        codes, scales = synth.fp8_weights(N, K, 2500)
    else:
        fmt, N, K, Ms, (codes, scales) = U.config_inputs(name)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    p = wq.wq_query_w8a8_plan(M, N, K, cu, True)
    U.note("w8a8 %s M=%d bands %s" % (name, M, p))
    if p["tail"] is None:
        pytest.skip("one band on a device of %d CUs" % cu)
    na = p["band"]
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(M, K, 2401 + M)
    xq, xc, xs = quantize(xb, K)
    y, _ = run(packed, N, K, xq, M, ws="auto")
    U.note("  one band, K whole")
    y1, _ = run(packed, N, K, xq, M)
    assert np.array_equal(y[:, :na], y1[:, :na])
    U.note("  one band, one K part")
    wq.wq_set_kparts(1)
    try:
        assert wq.wq_query_w8a8_plan(M, N, K, cu, False)["tail"] is None
        assert np.array_equal(run(packed, N, K, xq, M)[0], y1)
    finally:
        wq.wq_set_kparts(0)
    U.note("  the remaining columns alone")
    q = wq.wq_query_w8a8_plan(M, N - na, K, cu, True)
    assert q["tail"] is None and q["tile"] + (q["kparts"],) == p["tail"]
    pt = U.pack_fp8(np.ascontiguousarray(codes[na:]), np.ascontiguousarray(scales[na // 128:]))
    yt, _ = run(pt, N - na, K, xq, M, ws="auto")
    assert np.array_equal(y[:, na:], yt)
    assert np.array_equal(run(packed, N, K, xq, M, ws="auto")[0], y)
    cols = np.unique(np.concatenate([U.sample_cols(N, 72 + M, 192), np.arange(na - 16, na + 16)]))
    rows = np.arange(min(M, 4096 * 5120 // K))        # FFN down: the first 1204 rows
    y64 = oracle.gemm_w8a8(xc[rows], xs[rows], codes, scales, cols=cols)
    r = compare.grade(y[rows][:, cols], y64, floor_w8a8(xc[rows], xs[rows], codes, scales, K), "bf16")
    U.note("  %s" % r)
    check_w8a8(r)


def test_w8a8_streaming_tile_bits(kparts_reset):
    """The weight-streaming tile with one K group runs the tile kernel's
    arithmetic: FFN down in 4 K parts at M = 48 (streaming tile, 5
    column-waves) equals the first 48 rows of M = 128 in 4 parts (128 x 128
    tiles) bit for bit, NaN-filled workspaces both; and M = 48 against the
    oracle on sampled columns."""
    wq = U.wqmod()
    fmt, N, K, Ms, (codes, scales) = U.config_inputs("down")
    wq.wq_set_kparts(4)
    assert wq.wq_query_w8a8_plan(48, N, K, 256, True)["streaming"]
    assert not wq.wq_query_w8a8_plan(128, N, K, 256, True)["streaming"]
    packed = U.pack_fp8(codes, scales)
    xb = synth.x_bf16(128, K, 2301)
    xq, xc, xs = quantize(xb, K)
    U.note("w8a8 down M=128 in 4 parts (tile kernel)")
    ybig, _ = run(packed, N, K, xq, 128, ws="auto")
    U.note("w8a8 down M=48 in 4 parts (streaming tile)")
    xq48, xc48, xs48 = quantize(xb[:48], K)
    y, _ = run(packed, N, K, xq48, 48, ws="auto")
    assert np.array_equal(y, ybig[:48])
    cols = U.sample_cols(N, 71, 256)
    y64 = oracle.gemm_w8a8(xc48, xs48, codes, scales, cols=cols)
    check_w8a8(compare.grade(y[:, cols], y64, floor_w8a8(xc48, xs48, codes, scales, K), "bf16"))


def test_w8a8_workspace_errors(kparts_reset):
    wq = U.wqmod()
    wq.wq_set_kparts(3)
    N, K, M = 384, 1024, 40
    codes, scales = synth.fp8_weights(N, K, 1700)
    packed = U.pack_fp8(codes, scales)
    xq, _, _ = quantize(synth.x_bf16(M, K, 1701), K)
    need = wq.wq_w8a8_workspace_bytes(M, N, K)
    assert need == 3 * M * N * 4
    big = torch.zeros(need + 64, dtype=torch.uint8, device=U.DEV)
    y = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=U.DEV)
    with pytest.raises(wq.WqError) as e:
        wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, big[:need - 4])
    assert e.value.status == 4
    with pytest.raises(wq.WqError) as e:
        wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, big[8:8 + need])
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((y.float() == 5.0).all())


@pytest.mark.parametrize("ws", [True, False])
def test_w8a8_graph_replay_with_bands(ws):
    """Quantiser and a GEMM in two column bands (on 256 CUs: the leading band,
    the rest of the columns, and with a workspace their parts sum) captured in
    a HIP graph replay to the eager result, with eager work between replays."""
    wq = U.wqmod()
    N, K, M = 16640, 4096, 897
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    U.note("w8a8 graph replay with bands %s" % wq.wq_query_w8a8_plan(M, N, K, cu, ws))
    if cu == 256:
        assert wq.wq_query_w8a8_plan(M, N, K, cu, ws)["tail"] is not None
    codes, scales = synth.fp8_weights(N, K, 1810)
    packed = U.pack_fp8(codes, scales)
    x = U.t_u16(synth.x_bf16(M, K, 1811), torch.bfloat16)
    xq = torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=U.DEV)
    nb = wq.wq_w8a8_workspace_bytes(M, N, K) if ws else 0
    wsb = torch.empty(max(nb, 16), dtype=torch.uint8, device=U.DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_quantize_x_fp8(x, M, K, xq)
    wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, wsb if nb else None)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            wq.wq_quantize_x_fp8(x, M, K, xq)
            wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, wsb if nb else None)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.fill_(3.0)
        wsb.fill_(0xFF)
        xq.fill_(0x11)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep


def test_w8a8_graph_replay_with_parts(kparts_reset):
    """Quantiser, split GEMM and parts sum captured in a HIP graph replay to the eager result."""
    wq = U.wqmod()
    wq.wq_set_kparts(4)
    U.note("w8a8 graph replay with parts")
    N, K, M = 512, 2048, 96
    codes, scales = synth.fp8_weights(N, K, 1800)
    packed = U.pack_fp8(codes, scales)
    x = U.t_u16(synth.x_bf16(M, K, 1801), torch.bfloat16)
    xq = torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=U.DEV)
    ws = torch.empty(wq.wq_w8a8_workspace_bytes(M, N, K), dtype=torch.uint8, device=U.DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_quantize_x_fp8(x, M, K, xq)
    wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, ws)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            wq.wq_quantize_x_fp8(x, M, K, xq)
            wq.wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.fill_(3.0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep
