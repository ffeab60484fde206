"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

* dequant: the unpack hooks run the GEMM's own device dequant and must match the
  oracle bit for bit (every E4M3 code, every LUT code, FP16-subnormal products);
* GEMM: every output within 2 BF16 ULP of the oracle rounded to BF16, or within
  1e-3*sqrt(K)*max|x|*max|w| of it, on shapes that span several tiles and column
  groups with ragged tails, every M from 1 to 32, both FP8 paths;
* integer-exact inputs: the GPU result equals the exact integer rounded to BF16;
* invariants: power-of-two scale linearity, M=32 = two M=16 halves, GEMV rows =
  M=1 calls, MFMA rows = the M=16 call, determinism over repeats, strides and
  canaries, workspace left zeroed, pack determinism;
* the dense 3-bit LUT layout passes every LUT test and gives the nibble
  layout's GEMM bits exactly;
* special values: NaN weight codes and infinite or NaN activations give NaN
  and infinities exactly where the oracle's sum has them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import gpu_util as U

pytestmark = pytest.mark.gpu

AUTO, GEMV, MFMA = 0, 1, 2


# ---------------------------------------------------------------- dequant

def test_unpack_fp8_every_code_bit_exact():
    wq = U.wqmod()
    N, K = 256, 512
    U.note("unpack fp8 %dx%d" % (N, K))
    codes = (np.arange(N * K, dtype=np.int64) * 7 % 256).astype(np.uint8).reshape(N, K)
    scales = np.full((N // 128, K // 128), 3.0, dtype=np.float32)
    packed = U.pack_fp8(codes, scales)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_unpack_fp8_block(packed, N, K, out)
    out32 = torch.empty((N, K), dtype=torch.float32, device=U.DEV)
    wq.wq_unpack_fp8_block_f32(packed, N, K, out32)
    torch.cuda.synchronize()
    ref = oracle.e4m3_value(codes)
    got = U.bits_of(out)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * N * K // 256
    assert np.array_equal(got[~nan], oracle.bf16_rne(ref[~nan]))
    assert np.all(np.isnan(oracle.bf16_value(got[nan])))
    g32 = out32.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(g32), nan)
    assert np.array_equal(g32[~nan], ref[~nan]) and np.array_equal(np.signbit(g32[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_unpack_lut3_bit_exact_including_subnormal_products(dense):
    wq = U.wqmod()
    N, K = 48, 512                       # 3 tiles: a ragged column group for 4-tile groups
    U.note("unpack lut3 %dx%d dense=%d" % (N, K, dense))
    rng = np.random.Generator(np.random.PCG64(5))
    codes = rng.integers(0, 8, size=(N, K), dtype=np.uint8)
    codes[0, :8] = np.arange(8)
    qmap = np.sort(rng.standard_normal(8).astype(np.float16))
    qmap[2] = np.float16(0.0)
    g = (rng.uniform(0.5, 1.0, size=(N, K // 128)) * np.ldexp(1.0, rng.integers(-20, 3, size=(N, K // 128))))
    g = g.astype(np.float16)
    packed = U.pack_lut3(codes, qmap.view(np.uint16), g.view(np.uint16), dense=dense)
    out = torch.empty((N, K), dtype=torch.float16, device=U.DEV)
    (wq.wq_unpack_lut3_dense if dense else wq.wq_unpack_lut3)(packed, N, K, out)
    torch.cuda.synchronize()
    ref = oracle.f16_rne(oracle.dequant_lut3(codes, qmap.view(np.uint16), g.view(np.uint16)))
    got = U.bits_of(out)
    assert np.array_equal(got, ref)
    assert np.sum((np.abs(ref.view(np.float16)) < np.float16(2.0 ** -14)) & (ref & 0x7FFF != 0)) > 0


def test_pack_is_deterministic_and_stride_free():
    N, K = 384, 640
    U.note("pack determinism")
    codes, scales = synth.fp8_weights(N, K, 41)
    a = U.pack_fp8(codes, scales).cpu().numpy()
    b = U.pack_fp8(codes, scales, ldw=K + 96).cpu().numpy()
    assert np.array_equal(a, b)
    assert np.array_equal(a[N * K:].view(np.float32).reshape(scales.shape), scales)
    c, q, g = synth.lut3_weights(80, 384, 42)
    p1 = U.pack_lut3(c, q, g).cpu().numpy()
    p2 = U.pack_lut3(c, q, g).cpu().numpy()
    assert np.array_equal(p1, p2)
    d1 = U.pack_lut3(c, q, g, dense=True).cpu().numpy()
    d2 = U.pack_lut3(c, q, g, dense=True).cpu().numpy()
    assert np.array_equal(d1, d2)
    # the two layouts share everything after the codes: scales, map, status
    assert d1.size == p1.size - 80 * 384 // 8
    assert np.array_equal(d1[80 * 384 * 3 // 8:], p1[80 * 384 // 2:])


@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_pack_lut3_rejects_code_above_7(dense):
    wq = U.wqmod()
    U.note("pack lut3 bad code dense=%d" % dense)
    c, q, g = synth.lut3_weights(32, 256, 43)
    for bad in (8, 9, 255):               # 8: the 3-bit field itself is 0 -- still rejected
        c2 = c.copy()
        c2[17, 200] = bad
        with pytest.raises(wq.WqError) as e:
            U.pack_lut3(c2, q, g, dense=dense)
        assert e.value.status == 5
    U.pack_lut3(c, q, g, dense=dense)      # a valid matrix after a rejected one packs cleanly


# ------------------------------------------------------------------- GEMM

FP8_SHAPES = [(256, 512), (384, 1024), (1024, 640), (640, 2048)]


@pytest.mark.parametrize("N,K", FP8_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13, 16, 17, 24, 32])
def test_gemm_fp8_parity(N, K, M):
    U.note("fp8 parity N=%d K=%d M=%d" % (N, K, M))
    codes, scales = synth.fp8_weights(N, K, 100 + N + K)
    xbits = synth.x_bf16(M, K, 200 + M)
    packed = U.pack_fp8(codes, scales)
    paths = [AUTO, MFMA] + ([GEMV] if M <= 4 else [])
    for path in paths:
        y, _ = U.run_fp8(packed, N, K, xbits, path=path)
        r = U.grade_fp8(y, xbits, codes, scales, K)
        U.check(r, "path %d" % path)


@pytest.fixture
def kparts_reset():
    yield
    U.wqmod().wq_set_kparts(0)


@pytest.mark.parametrize("N", [128, 256])
def test_fp8_single_k_block(N, kparts_reset):
    """The smallest legal shapes: one 128-wide K block (K groups and K parts
    have nothing to split) and one or two 128-row scale blocks; every path,
    with and without a workspace, forced part counts clamped to one block."""
    wq = U.wqmod()
    K = 128
    U.note("fp8 single K block N=%d" % N)
    codes, scales = synth.fp8_weights(N, K, 940 + N)
    packed = U.pack_fp8(codes, scales)
    for M in (1, 2, 4, 5, 16, 17, 32):
        xbits = synth.x_bf16(M, K, 941 + M)
        for path in [AUTO, MFMA] + ([GEMV] if M <= 4 else []):
            for kp in (0, 4):
                wq.wq_set_kparts(kp)
                for ws in (None, "auto"):
                    y, _ = U.run_fp8(packed, N, K, xbits, path=path, ws=ws)
                    U.check(U.grade_fp8(y, xbits, codes, scales, K), "M=%d path=%d kp=%d ws=%s" % (M, path, kp, ws))
        wq.wq_set_kparts(0)


LUT_SHAPES = [(48, 256), (272, 1024), (1024, 384), (528, 2048)]


@pytest.mark.parametrize("N,K", LUT_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 4, 7, 16, 20, 32])
@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_gemm_lut3_parity(N, K, M, dense):
    U.note("lut3 parity N=%d K=%d M=%d dense=%d" % (N, K, M, dense))
    c, q, g = synth.lut3_weights(N, K, 300 + N + K)
    xbits = synth.x_f16(M, K, 400 + M)
    packed = U.pack_lut3(c, q, g, dense=dense)
    y, _ = U.run_lut3(packed, N, K, xbits, dense=dense)
    r = U.grade_lut3(y, xbits, c, q, g, K)
    U.check(r, out_dtype="f16")


@pytest.mark.parametrize("K", [128, 640, 1664])
@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_lut3_partial_quads(K, dense):
    """K blocks not a multiple of 4 (one block; a quad plus one; 13 blocks over
    two K groups): the lanes whose block of the last quad lies past K load
    zeros, every M from 1 to 32 passes the oracle."""
    N = 112
    U.note("lut3 partial quads K=%d dense=%d" % (K, dense))
    c, q, g = synth.lut3_weights(N, K, 930 + K)
    packed = U.pack_lut3(c, q, g, dense=dense)
    for M in (1, 3, 16, 17, 32):
        xh = synth.x_f16(M, K, 931 + M)
        y, _ = U.run_lut3(packed, N, K, xh, dense=dense)
        r = U.grade_lut3(y, xh, c, q, g, K)
        U.check(r, "K=%d M=%d" % (K, M), "f16")


@pytest.mark.parametrize("N,K", [(48, 256), (528, 2048), (1024, 1152)])
def test_dense_lut3_gives_the_nibble_bits(N, K):
    """The two storage layouts feed the same decode and the same arithmetic, so
    the GEMM outputs agree bit for bit for every M (both 16-row halves too)."""
    U.note("lut3 dense == nibble N=%d K=%d" % (N, K))
    c, q, g = synth.lut3_weights(N, K, 900 + N)
    pn, pd = U.pack_lut3(c, q, g), U.pack_lut3(c, q, g, dense=True)
    x32 = synth.x_f16(32, K, 901)
    for M in (1, 3, 8, 16, 17, 32):
        yn, _ = U.run_lut3(pn, N, K, x32[:M])
        yd, _ = U.run_lut3(pd, N, K, x32[:M], dense=True)
        assert np.array_equal(yn, yd), M


def test_integer_exact_results_are_exact():
    U.note("integer exact")
    rng = np.random.Generator(np.random.PCG64(44))
    N, K, M = 256, 1024, 16
    wi = rng.integers(-8, 9, size=(N, K))
    xi = rng.integers(-2, 3, size=(M, K))
    codes = torch.from_numpy(wi.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = np.ones((N // 128, K // 128), dtype=np.float32)
    xbits = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    exact = oracle.bf16_rne((xi @ wi.T).astype(np.float64))
    packed = U.pack_fp8(codes, scales)
    for M_ in (1, 4, 16):
        for path in ([GEMV, MFMA] if M_ <= 4 else [MFMA]):
            y, _ = U.run_fp8(packed, N, K, xbits[:M_], path=path)
            assert np.array_equal(y, exact[:M_]), (M_, path)
    ci = rng.integers(0, 8, size=(N, K)).astype(np.uint8)
    qmap = np.arange(-4, 4).astype(np.float16).view(np.uint16)
    g = np.ones((N, K // 128), dtype=np.float16).view(np.uint16)
    xh = xi.astype(np.float16).view(np.uint16)
    exact_l = oracle.f16_rne((xi @ (ci.astype(np.int64) - 4).T).astype(np.float64))
    for dense in (False, True):
        yl, _ = U.run_lut3(U.pack_lut3(ci, qmap, g, dense=dense), N, K, xh, dense=dense)
        assert np.array_equal(yl, exact_l), dense


@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_lut3_subnormal_weights_are_exact(dense):
    """Map {-4..3} and every group scale 2^-24 (FP16 bits 0x0001): each
    dequantised weight q * 2^-24 is an exact FP16 subnormal, and the FP16
    matrix core must take it unflushed.  With x in {-2..2} every product and
    every partial sum is an integer times 2^-24 (|sum| < 2^24), exact in FP32
    in any order, so each output must be fp16_rne(exact) bit for bit; the
    oracle's binary64 sum is the exact value itself.  K = 1152 ends in a
    partial quad of K blocks; M = 20 and 32 take the 32-row pass."""
    N, K = 272, 1152
    U.note("lut3 subnormal weights dense=%d" % dense)
    rng = np.random.Generator(np.random.PCG64(1701))
    ci = rng.integers(0, 8, size=(N, K)).astype(np.uint8)
    qmap = np.arange(-4, 4).astype(np.float16).view(np.uint16)
    g = np.full((N, K // 128), 0x0001, dtype=np.uint16)
    wq = U.wqmod()
    packed = U.pack_lut3(ci, qmap, g, dense=dense)
    w = torch.empty((N, K), dtype=torch.float16, device=U.DEV)
    (wq.wq_unpack_lut3_dense if dense else wq.wq_unpack_lut3)(packed, N, K, w)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.f16_value(U.bits_of(w)), (ci.astype(np.int64) - 4) * 2.0 ** -24)
    for M in (1, 5, 16, 20, 32):
        xi = rng.integers(-2, 3, size=(M, K))
        xh = xi.astype(np.float16).view(np.uint16)
        S = xi @ (ci.astype(np.int64) - 4).T
        exact = S.astype(np.float64) * 2.0 ** -24
        y, _ = U.run_lut3(packed, N, K, xh, dense=dense)
        assert np.array_equal(y, oracle.f16_rne(exact)), M
        assert np.array_equal(oracle.gemm_lut3(xh, ci, qmap, g), exact), M


def test_fp8_subnormal_activations_are_exact():
    """BF16-subnormal activations x = j * 2^-133 (|j| <= 127) against E4M3
    weights that are small integers, block scale 2^110: every product and
    every 128-K block sum is an integer times 2^-133, an FP32 number exactly
    (FP32 subnormals reach 2^-149), the fold times 2^110 is exact and the
    output S * 2^-23 (|S| < 2^24) is a BF16 normal.  The matrix core and the
    GEMV must take the subnormal operands unflushed: every output equals
    bf16_rne(exact) bit for bit on every path, with and without K parts."""
    N, K = 256, 1024
    U.note("fp8 subnormal activations")
    rng = np.random.Generator(np.random.PCG64(1702))
    wi = rng.integers(-8, 9, size=(N, K))
    codes = oracle.e4m3_rne(wi.astype(np.float32))
    assert np.array_equal(oracle.e4m3_value(codes), wi)
    scales = np.full((N // 128, K // 128), 2.0 ** 110, dtype=np.float32)
    packed = U.pack_fp8(codes, scales)
    wq = U.wqmod()
    for M in (1, 4, 16, 32):
        xi = rng.integers(-127, 128, size=(M, K))
        xbits = (np.abs(xi) | np.where(xi < 0, 0x8000, 0)).astype(np.uint16)
        assert np.array_equal(oracle.bf16_value(xbits), xi * 2.0 ** -133)
        exact = (xi @ wi.T).astype(np.float64) * 2.0 ** -23
        want = oracle.bf16_rne(exact)
        assert np.array_equal(oracle.gemm_fp8(xbits, codes, scales), exact), M
        for path in ([GEMV, MFMA] if M <= 4 else [MFMA]):
            for kp in (0, 3):
                wq.wq_set_kparts(kp)
                try:
                    y, _ = U.run_fp8(packed, N, K, xbits, path=path, ws="auto" if kp else None)
                finally:
                    wq.wq_set_kparts(0)
                assert np.array_equal(y, want), (M, path, kp)


def test_invariants_fp8():
    U.note("invariants fp8")
    N, K = 640, 1280
    codes, scales = synth.fp8_weights(N, K, 45)
    x32 = synth.x_bf16(32, K, 46)
    packed = U.pack_fp8(codes, scales)
    packed2 = U.pack_fp8(codes, scales * np.float32(2.0))
    y32, _ = U.run_fp8(packed, N, K, x32, path=MFMA)
    # scale linearity (bitwise): doubling every block scale doubles every output
    y32b, _ = U.run_fp8(packed2, N, K, x32, path=MFMA)
    v1, v2 = oracle.bf16_value(y32), oracle.bf16_value(y32b)
    assert np.array_equal(v2, 2 * v1)
    # M=32 is two M=16 halves
    ya, _ = U.run_fp8(packed, N, K, x32[:16], path=MFMA)
    yb, _ = U.run_fp8(packed, N, K, x32[16:], path=MFMA)
    assert np.array_equal(np.vstack([ya, yb]), y32)
    # MFMA rows of an M-call equal those rows of the M=16 call
    for M in (5, 9, 13):
        yM, _ = U.run_fp8(packed, N, K, x32[:M], path=MFMA)
        assert np.array_equal(yM, ya[:M]), M
    # GEMV rows of an M-call equal the M=1 calls of those rows
    ones = [U.run_fp8(packed, N, K, x32[m:m + 1], path=GEMV)[0] for m in range(4)]
    for M in (2, 3, 4):
        yM, _ = U.run_fp8(packed, N, K, x32[:M], path=GEMV)
        assert np.array_equal(yM, np.vstack(ones[:M])), M
    # determinism over repeats, sharing one workspace across paths
    wq = U.wqmod()
    ws = wq.workspace(wq.WQ_FMT_FP8_BLOCK, N, K, U.DEV)
    for i in range(20):
        path = (MFMA, GEMV)[i % 2]
        xs = x32[:16] if path == MFMA else x32[:4]
        yr, _ = U.run_fp8(packed, N, K, xs, path=path, ws=ws)
        assert np.array_equal(yr, ya if path == MFMA else np.vstack(ones[:4])), i


@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_invariants_lut3(dense):
    U.note("invariants lut3 dense=%d" % dense)
    N, K = 528, 1024
    c, q, g = synth.lut3_weights(N, K, 47)
    # doubling the group scales doubles every dequantised weight exactly only
    # while no product qmap[c]*g is an FP16 subnormal: keep map entries >= 0.02
    qf = q.view(np.float16).astype(np.float32)
    q = np.where(np.abs(qf) < 0.02, np.copysign(0.02, qf), qf).astype(np.float16).view(np.uint16)
    assert (np.abs(q.view(np.float16).astype(np.float64)).min() * g.view(np.float16).astype(np.float64).min()
            >= 2.0 ** -14)
    x32 = synth.x_f16(32, K, 48)
    packed = U.pack_lut3(c, q, g, dense=dense)
    g2 = (g.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    y32, _ = U.run_lut3(packed, N, K, x32, dense=dense)
    y32b, _ = U.run_lut3(U.pack_lut3(c, q, g2, dense=dense), N, K, x32, dense=dense)
    v1, v2 = oracle.f16_value(y32), oracle.f16_value(y32b)
    # exact where the FP16 output is normal; an output that cancelled into the
    # FP16 subnormal range is rounded on a fixed 2^-24 grid, so there doubling
    # the exact sum and rounding may differ from rounding then doubling by one step
    normal = np.abs(v1) >= 2.0 ** -14
    assert np.array_equal(v2[normal], 2 * v1[normal])
    assert np.all(np.abs(v2[~normal] - 2 * v1[~normal]) <= 2.0 ** -24)
    ya, _ = U.run_lut3(packed, N, K, x32[:16], dense=dense)
    yb, _ = U.run_lut3(packed, N, K, x32[16:], dense=dense)
    assert np.array_equal(np.vstack([ya, yb]), y32)
    for M in (1, 2, 7, 15):
        yM, _ = U.run_lut3(packed, N, K, x32[:M], dense=dense)
        assert np.array_equal(yM, ya[:M]), M
    wq = U.wqmod()
    ws = wq.workspace(wq.WQ_FMT_LUT3_DENSE if dense else wq.WQ_FMT_LUT3, N, K, U.DEV)
    for i in range(20):
        yr, _ = U.run_lut3(packed, N, K, x32[:16], ws=ws, dense=dense)
        assert np.array_equal(yr, ya), i


def test_strides_and_canaries():
    U.note("strides and canaries")
    N, K, M = 384, 768, 20
    codes, scales = synth.fp8_weights(N, K, 49)
    packed = U.pack_fp8(codes, scales)
    xs = synth.x_bf16(M, K, 50, ld=K + 40)            # NaN canaries in the x padding
    ldy = N + 24
    canary = np.full((M, ldy), 0x7FAB, dtype=np.uint16)
    for path in (AUTO, MFMA):
        y, full = U.run_fp8(packed, N, K, xs, path=path, ldy=ldy, y_init=canary)
        U.check(U.grade_fp8(y, xs, codes, scales, K), "path %d" % path)
        assert np.all(full[:, N:] == 0x7FAB)
    y4, full4 = U.run_fp8(packed, N, K, xs[:4], path=GEMV, ldy=ldy, y_init=canary[:4])
    U.check(U.grade_fp8(y4, xs[:4], codes, scales, K), "gemv")
    assert np.all(full4[:, N:] == 0x7FAB)
    c, q, g = synth.lut3_weights(N, K, 51)
    xh = synth.x_f16(M, K, 52, ld=K + 8)
    for dense in (False, True):
        yl, fl = U.run_lut3(U.pack_lut3(c, q, g, dense=dense), N, K, xh, ldy=ldy, y_init=canary, dense=dense)
        U.check(U.grade_lut3(yl, xh, c, q, g, K), "dense=%d" % dense, "f16")
        assert np.all(fl[:, N:] == 0x7FAB), dense


def test_zero_rows_and_zero_matrix():
    U.note("degenerate inputs")
    N, K = 256, 512
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.ones((N // 128, K // 128), dtype=np.float32)
    xbits = synth.x_bf16(8, K, 53)
    for path in (MFMA, GEMV):
        y, _ = U.run_fp8(U.pack_fp8(codes, scales), N, K, xbits[: (8 if path == MFMA else 4)], path=path)
        assert not (y & 0x7FFF).any()


def test_nan_codes_poison_exactly_their_columns():
    """E4M3 NaN codes (0x7F, 0xFF) in W: every output of a column whose row
    of W holds one is NaN on every path (GEMV, MFMA tile, K parts across
    work-groups, 32-row single pass), every other output is finite and passes
    the oracle."""
    U.note("nan codes")
    N, K = 512, 2048
    codes, scales = synth.fp8_weights(N, K, 57)
    codes = codes.copy()
    bad = [3, 130, 257, 511]
    for i, n in enumerate(bad):
        codes[n, (97 * i + 5) % K] = 0x7F if i % 2 == 0 else 0xFF
    packed = U.pack_fp8(codes, scales)
    wq = U.wqmod()
    for path, M in ((GEMV, 1), (GEMV, 4), (MFMA, 16), (MFMA, 32)):
        for ws in (None, "auto"):
            wq.wq_set_kparts(4 if ws else 0)
            try:
                xbits = synth.x_bf16(M, K, 58)
                y, _ = U.run_fp8(packed, N, K, xbits, path=path, ws=ws)
            finally:
                wq.wq_set_kparts(0)
            nan = np.isnan(oracle.bf16_value(y))
            expect = np.zeros(N, dtype=bool)
            expect[bad] = True
            assert np.array_equal(nan, np.broadcast_to(expect, nan.shape)), (path, M, ws)
            ok = ~expect
            y64 = oracle.gemm_fp8(xbits, codes, scales, K=K)
            assert np.all(np.isnan(y64[:, expect])) and np.all(np.isfinite(y64[:, ok]))
            g = U.compare.grade(y, y64, U.floor_fp8(xbits, codes, scales, K), "bf16")
            U.check(g, "path %d M=%d ws=%s" % (path, M, ws))


def _check_nonfinite(yv, y64, ybits, floor, out_dtype, what):
    """NaN exactly where the oracle's sum is NaN, infinities with the oracle's
    sign, every finite output graded against the oracle."""
    assert np.array_equal(np.isnan(yv), np.isnan(y64)), what
    assert np.array_equal(np.isposinf(yv), np.isposinf(y64)), what
    assert np.array_equal(np.isneginf(yv), np.isneginf(y64)), what
    fin = np.isfinite(y64)
    g = U.compare.grade(ybits[fin], y64[fin], floor, out_dtype)
    U.check(g, str(what), out_dtype)


def test_nonfinite_activations_follow_ieee():
    """Infinite and NaN activations (BF16 for FP8 weights, FP16 for the LUT):
    an infinity times a nonzero weight is an infinity of the product's sign, an
    infinity times a zero weight (an E4M3 +0/-0 code, a zero group scale) and
    opposite infinities in one sum are NaN, a NaN activation makes its row NaN,
    on every path (GEMV, MFMA tile, K parts across work-groups, the 32-row
    single pass); the oracle decides each output's class."""
    U.note("non-finite activations")
    wq = U.wqmod()
    N, K = 512, 2048
    codes, scales = synth.fp8_weights(N, K, 61)
    codes = codes.copy()
    codes[7, 100] = 0x00          # +0 and -0 weights under the row-0 infinity
    codes[300, 100] = 0x80
    specials = {(0, 100): 0x7F80, (1, 700): 0x7FC0, (2, 5): 0x7F80, (2, 1500): 0xFF80, (3, 2047): 0xFF80}
    packed = U.pack_fp8(codes, scales)
    for path, M in ((GEMV, 1), (GEMV, 4), (MFMA, 5), (MFMA, 16), (MFMA, 32)):
        xbits = synth.x_bf16(M, K, 62).copy()
        fin_x = xbits.copy()
        for (m, k), b in specials.items():
            if m < M:
                xbits[m, k] = b
                fin_x[m, k] = 0
        y64 = oracle.gemm_fp8(xbits, codes, scales, K=K)
        assert np.isnan(y64[0, [7, 300]]).all() and np.isinf(y64[0, 0])
        floor = U.floor_fp8(fin_x, codes, scales, K)
        for ws in (None, "auto"):
            wq.wq_set_kparts(4 if ws else 0)
            try:
                y, _ = U.run_fp8(packed, N, K, xbits, path=path, ws=ws)
            finally:
                wq.wq_set_kparts(0)
            _check_nonfinite(oracle.bf16_value(y), y64, y, floor, "bf16", ("fp8", path, M, ws))

    N, K = 528, 1152
    codes, qmap, g = synth.lut3_weights(N, K, 63)
    g = g.copy()
    g[9, 0] = 0                   # a zero group scale under the row-0 infinity
    lut_specials = {(0, 100): 0x7C00, (1, 700): 0x7E00, (2, 5): 0x7C00, (2, 1000): 0xFC00, (3, 1151): 0xFC00}
    for dense in (False, True):
        packed = U.pack_lut3(codes, qmap, g, dense=dense)
        for M in (1, 4, 16, 17, 32):
            xbits = synth.x_f16(M, K, 64).copy()
            fin_x = xbits.copy()
            for (m, k), b in lut_specials.items():
                if m < M:
                    xbits[m, k] = b
                    fin_x[m, k] = 0
            y64 = oracle.gemm_lut3(xbits, codes, qmap, g, K=K)
            assert np.isnan(y64[0, 9]) and np.isinf(y64[0, 0])
            floor = U.floor_lut3(fin_x, codes, qmap, g, K)
            y, _ = U.run_lut3(packed, N, K, xbits, dense=dense)
            _check_nonfinite(oracle.f16_value(y), y64, y, floor, "f16", ("lut3", dense, M))


# ------------------------------------------------------ every kernel variant

# (nt, sn, split): every activation-piece count per lane the kernels are built
# for (sn = 1, 2, 3, 4/5, 6/7, 8), one to four K groups, 1- and 2-tile waves,
# and the 16-wave work-groups of the one-tile LUT kernels (FP8 clamps to 8)
TUNINGS = [(1, 1, 1), (1, 1, 4), (2, 1, 3), (1, 2, 4), (2, 2, 8), (1, 3, 6), (2, 3, 6), (1, 4, 4),
           (1, 4, 8), (2, 4, 8), (1, 5, 5), (1, 6, 6), (1, 7, 7), (2, 7, 7), (1, 8, 8), (2, 8, 8),
           (1, 4, 16), (1, 7, 14)]


@pytest.fixture
def tuning_reset():
    yield
    U.wqmod().wq_set_tuning(0, 0, 0, 0)


@pytest.mark.parametrize("nt,sn,split", TUNINGS, ids=["nt%d-sn%d-s%d" % t for t in TUNINGS])
def test_every_tiling_matches_oracle(nt, sn, split, tuning_reset):
    """Ragged column groups (tiles past N inside a group), K ranges of unequal
    length, and M on both sides of 8 and 16, for each tiling."""
    wq = U.wqmod()
    wq.wq_set_tuning(nt, sn, split, 0)
    U.note("tiling nt=%d sn=%d split=%d" % (nt, sn, split))
    for N, K in ((384, 1152), (640, 640)):
        codes, scales = synth.fp8_weights(N, K, 500 + N)
        packed = U.pack_fp8(codes, scales)
        for M in (1, 5, 16, 20):
            xbits = synth.x_bf16(M, K, 600 + M)
            y, _ = U.run_fp8(packed, N, K, xbits, path=MFMA)
            r = U.grade_fp8(y, xbits, codes, scales, K)
            U.check(r, "fp8 N=%d K=%d M=%d" % (N, K, M))
        for M in (1, 3):   # the GEMV takes the same (sn, split); it always runs one tile per wave
            xbits = synth.x_bf16(M, K, 650 + M)
            y, _ = U.run_fp8(packed, N, K, xbits, path=GEMV)
            r = U.grade_fp8(y, xbits, codes, scales, K)
            U.check(r, "fp8 gemv N=%d K=%d M=%d" % (N, K, M))
    for N, K in ((48, 384), (272, 1152)):
        c, q, g = synth.lut3_weights(N, K, 700 + N)
        packed = U.pack_lut3(c, q, g)
        packed_d = U.pack_lut3(c, q, g, dense=True)
        for M in (1, 7, 16, 24):
            xh = synth.x_f16(M, K, 800 + M)
            y, _ = U.run_lut3(packed, N, K, xh)
            r = U.grade_lut3(y, xh, c, q, g, K)
            U.check(r, "lut3 N=%d K=%d M=%d" % (N, K, M), "f16")
            yd, _ = U.run_lut3(packed_d, N, K, xh, dense=True)
            assert np.array_equal(yd, y), "lut3 dense N=%d K=%d M=%d" % (N, K, M)


# Tilings whose 32-row LUT chunks fit, so M = 17..32 runs in one pass with
# both 16-row halves fed by each dequantised operand (the host's single-pass
# rule: 4, 5, 6 or 8 activation pieces per lane within the launch bound, and
# the K groups' double-buffered 32-row chunks within LDS), and two that do
# not (16 pieces per lane; 16 pieces and 4 K groups).
LUT_SINGLE_PASS = [(1, 8, 8), (1, 8, 16), (1, 6, 6), (1, 4, 8), (1, 7, 14), (1, 2, 4), (1, 2, 8)]


@pytest.mark.parametrize("nt,sn,split", LUT_SINGLE_PASS, ids=["sn%d-s%d" % t[1:] for t in LUT_SINGLE_PASS])
@pytest.mark.parametrize("dense", [False, True], ids=["nibble", "dense"])
def test_lut3_single_pass_rows_equal_16_row_calls(nt, sn, split, dense, tuning_reset):
    """A 32-row LUT call (one pass or two) gives each row the bits of the
    16-row call holding that row, and passes the oracle; K = 1152 ends in a
    partial quad of K blocks."""
    wq = U.wqmod()
    wq.wq_set_tuning(nt, sn, split, 0)
    U.note("lut3 single pass sn=%d split=%d dense=%d" % (sn, split, dense))
    N, K = 400, 1152
    c, q, g = synth.lut3_weights(N, K, 910)
    packed = U.pack_lut3(c, q, g, dense=dense)
    x32 = synth.x_f16(32, K, 911)
    y32, _ = U.run_lut3(packed, N, K, x32, dense=dense)
    ya, _ = U.run_lut3(packed, N, K, x32[:16], dense=dense)
    yb, _ = U.run_lut3(packed, N, K, x32[16:], dense=dense)
    assert np.array_equal(y32, np.vstack([ya, yb]))
    y20, _ = U.run_lut3(packed, N, K, x32[:20], dense=dense)
    assert np.array_equal(y20, y32[:20])
    r = U.grade_lut3(y32, x32, c, q, g, K)
    U.check(r, out_dtype="f16")


def test_hip_graph_replays_match_eager():
    """The GEMM captured in a HIP graph (no memset nodes: the library queues
    kernels only) replays to the eager result every time, with eager work and
    synchronisations between the replays."""
    wq = U.wqmod()
    U.note("hip graph replay")
    N, K, M = 640, 1280, 16
    codes, scales = synth.fp8_weights(N, K, 90)
    packed = U.pack_fp8(codes, scales)
    x = U.t_u16(synth.x_bf16(M, K, 91), torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)
    c, q, g = synth.lut3_weights(N, K, 92)
    pl = U.pack_lut3(c, q, g)
    pd = U.pack_lut3(c, q, g, dense=True)
    xh = U.t_u16(synth.x_f16(M, K, 93), torch.float16)
    yl = torch.empty((M, N), dtype=torch.float16, device=U.DEV)
    yd = torch.empty((M, N), dtype=torch.float16, device=U.DEV)
    wq.wq_gemm_fp8_block(packed, N, K, x, y, M)
    wq.wq_gemm_lut3(pl, N, K, xh, yl, M)
    wq.wq_gemm_lut3_dense(pd, N, K, xh, yd, M)
    torch.cuda.synchronize()
    ref, refl, refd = y.clone(), yl.clone(), yd.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            wq.wq_gemm_fp8_block(packed, N, K, x, y, M)
            wq.wq_gemm_lut3(pl, N, K, xh, yl, M)
            wq.wq_gemm_lut3_dense(pd, N, K, xh, yd, M)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.fill_(7.0)
        yl.fill_(7.0)
        yd.fill_(7.0)
        wq.wq_gemm_fp8_block_path(packed, N, K, x[:3], y[:3], 3, None, GEMV)   # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep
        assert torch.equal(yl.view(torch.int16), refl.view(torch.int16)), rep
        assert torch.equal(yd.view(torch.int16), refd.view(torch.int16)), rep
