"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with an
independent source:

* library decoders present here (``torch.float8_e4m3fn``, ``torch.bfloat16``,
  ``numpy.float16``) applied to every bit pattern of a format;
* published reference points of the formats (``tests/golden/``);
* brute force over every representable value for rounding (nearest finite value,
  ties to the even pattern, compared in exact rationals);
* exact rational sums (``fractions.Fraction``) of the GEMM on tiny shapes, with
  the weights decoded by the library decoders, not by the oracle;
* integer-exact special cases checked against numpy's int64 matmul;
* closed forms and invariants (power-of-two scale linearity, stride and canary
  independence, row/column independence, thread-count independence).

The mutation tests run these same functions against deliberately broken copies
of the oracle and require that every planted mistake trips at least one pin.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers

def _same_bits_f64(a: np.ndarray, b: np.ndarray) -> bool:
    """Equal values, equal signs of zero, NaN where NaN (payload free)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    if not np.array_equal(nan_a, nan_b):
        return False
    m = ~nan_a
    return bool(np.array_equal(a[m], b[m]) and np.array_equal(np.signbit(a[m]), np.signbit(b[m])))


def _torch_e4m3(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_bf16(bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _numpy_f16(bits) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _parse_value(tok: str) -> float | Fraction:
    if tok == "nan":
        return float("nan")
    if tok in ("inf", "-inf"):
        return float(tok)
    if tok == "-0":
        return -0.0
    return Fraction(Decimal(tok))


def _golden_rows(name: str):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def _all_finite(fmt: str):
    """All finite values of a 16-bit format, sorted, with their bit patterns (library decode)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = _numpy_f16(bits) if fmt == "f16" else _torch_bf16(bits)
    keep = np.isfinite(vals) & ~((vals == 0) & np.signbit(vals))
    vals, bits = vals[keep], bits[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


def _brute_round(v: float, vals: np.ndarray, bits: np.ndarray, inf_bits: int, overflow_at: Fraction) -> int:
    """Nearest representable value by exhaustive neighbour search, ties to even pattern."""
    if math.isnan(v):
        return -1
    fv = Fraction(v)
    if abs(fv) >= overflow_at:
        return inf_bits | (0x8000 if v < 0 else 0)
    i = int(np.searchsorted(vals, v))
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(vals)]
    best = None
    for j in cands:
        d = abs(fv - Fraction(float(vals[j])))
        key = (d, int(bits[j]) & 1)
        if best is None or key < best[0]:
            best = (key, int(bits[j]))
    out = best[1]
    if out == 0 and math.copysign(1.0, v) < 0:
        out = 0x8000  # a negative value that rounds to zero keeps its sign
    return out


def _rand_doubles(rng, n, lo_exp, hi_exp):
    mant = rng.uniform(1.0, 2.0, size=n)
    exps = rng.integers(lo_exp, hi_exp, size=n)
    sign = rng.choice([-1.0, 1.0], size=n)
    return sign * np.ldexp(mant, exps)


# ----------------------------------------------------------------- formats

def pin_e4m3_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    assert _same_bits_f64(oracle.e4m3_value(codes), _torch_e4m3(codes)), "E4M3 decode != torch"


def pin_e4m3_golden():
    for code, val in _golden_rows("e4m3_ocp_points.txt"):
        got = float(oracle.e4m3_value([int(code, 16)])[0])
        want = _parse_value(val)
        if isinstance(want, float) and math.isnan(want):
            assert math.isnan(got), code
        else:
            assert Fraction(got) == Fraction(want) and math.copysign(1, got) == math.copysign(1, float(want)), (code, got, val)


def pin_f16_decode_all():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _same_bits_f64(oracle.f16_value(bits), _numpy_f16(bits)), "FP16 decode != numpy"


def pin_bf16_decode_all():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _same_bits_f64(oracle.bf16_value(bits), _torch_bf16(bits)), "BF16 decode != torch"


def pin_16bit_golden():
    for fmt, b, val in _golden_rows("f16_bf16_points.txt"):
        bits = np.array([int(b, 16)], dtype=np.uint16)
        got = float((oracle.f16_value if fmt == "f16" else oracle.bf16_value)(bits)[0])
        want = _parse_value(val)
        if isinstance(want, float) and math.isnan(want):
            assert math.isnan(got), (fmt, b)
        elif isinstance(want, float) and math.isinf(want):
            assert got == want, (fmt, b)
        else:
            assert Fraction(got) == want, (fmt, b, got, val)
        # and the value rounds back to its own pattern
        if not (isinstance(want, float) and math.isnan(want)):
            back = (oracle.f16_rne if fmt == "f16" else oracle.bf16_rne)(np.array([got]))[0]
            assert int(back) == int(b, 16), (fmt, b, hex(int(back)))


def _rounding_inputs(fmt: str, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    vals, _ = _all_finite(fmt)
    lo, hi = ((-27, 17) if fmt == "f16" else (-136, 129))
    v = list(_rand_doubles(rng, 3000, lo, hi))
    # exact midpoints between neighbours (ties), and points just beside them
    idx = rng.integers(0, len(vals) - 1, size=600)
    for i in idx:
        a, b = float(vals[i]), float(vals[i + 1])
        mid = (a + b) / 2.0               # exact: both have few significant bits
        v += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    top = float(vals[-1])
    ulp_top = top - float(vals[-2])
    v += [top, top + ulp_top / 2, np.nextafter(top + ulp_top / 2, 0.0), top * 4, -top - ulp_top / 2,
          0.0, -0.0, float(vals[len(vals) // 2 + 1]) / 2, float("inf"), float("-inf")]
    return np.array(v, dtype=np.float64)


def _overflow_at(fmt: str) -> Fraction:
    vals, _ = _all_finite(fmt)
    top = Fraction(float(vals[-1]))
    ulp = top - Fraction(float(vals[-2]))
    return top + ulp / 2


def pin_f16_rne():
    v = _rounding_inputs("f16", 11)
    got = oracle.f16_rne(v)
    # (1) numpy's binary64 -> binary16 cast (correctly rounded)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), "f16_rne != numpy cast at %s" % v[np.argmax(got != want)]
    # (2) exhaustive nearest-value search on a subsample
    vals, bits = _all_finite("f16")
    ov = _overflow_at("f16")
    for x, g in list(zip(v, got))[::7]:
        if math.isinf(x):
            continue
        assert _brute_round(float(x), vals, bits, 0x7C00, ov) == int(g), (x, hex(int(g)))


def pin_bf16_rne():
    v = _rounding_inputs("bf16", 12)
    got = oracle.bf16_rne(v)
    vals, bits = _all_finite("bf16")
    ov = _overflow_at("bf16")
    for x, g in zip(v, got):
        if math.isinf(x):
            assert int(g) == (0x7F80 | (0x8000 if x < 0 else 0))
            continue
        assert _brute_round(float(x), vals, bits, 0x7F80, ov) == int(g), (x, hex(int(g)))
    # float32-representable inputs: torch's float32 -> bfloat16 cast is a single rounding
    f32 = v[np.isfinite(v) & (np.abs(v) < 3e38) & (np.abs(v) > 1e-37)].astype(np.float32)
    want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(f32.astype(np.float64)), want), "bf16_rne != torch on float32 inputs"


# ----------------------------------------------------------------- dequant

def pin_fp8_dequant():
    N, K = 256, 384
    codes = np.random.Generator(np.random.PCG64(21)).integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scales = np.array([[0.5, 3.0, 0.0078125], [1.75, 0.375, 96.0]], dtype=np.float32)
    want = _torch_e4m3(codes) * np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    assert _same_bits_f64(oracle.dequant_fp8(codes, scales), want), "FP8 dequant != torch decode * scale"


def pin_lut_dequant():
    rng = np.random.Generator(np.random.PCG64(22))
    N, K = 64, 512
    codes = rng.integers(0, 8, size=(N, K), dtype=np.uint8)
    qmap = np.sort(rng.standard_normal(8).astype(np.float16))
    qmap[3] = np.float16(0.0)
    # group scales spanning normal and tiny magnitudes so some products are FP16 subnormal
    g = (rng.uniform(0.5, 1.0, size=(N, K // 128)) * np.ldexp(1.0, rng.integers(-22, 2, size=(N, K // 128))))
    g = g.astype(np.float16)
    g[g == 0] = np.float16(2.0 ** -24)
    want = (qmap.astype(np.float64)[codes] * np.repeat(g.astype(np.float64), 128, 1)).astype(np.float16)
    got = oracle.dequant_lut3(codes, qmap.view(np.uint16), g.view(np.uint16))
    assert _same_bits_f64(got, want.astype(np.float64)), "LUT dequant != numpy float16(q*g)"
    n_sub = int(np.sum((np.abs(want) < np.float16(2.0 ** -14)) & (want != 0)))
    assert n_sub > 0, "fixture should exercise subnormal products"


def pin_lut_rejects_bad_code():
    codes = np.zeros((16, 128), dtype=np.uint8)
    codes[3, 5] = 8
    try:
        oracle.dequant_lut3(codes, np.zeros(8, np.uint16), np.zeros((16, 1), np.uint16))
    except ValueError:
        return
    raise AssertionError("code 8 accepted")


# -------------------------------------------------------------------- GEMM

def _exact_fp8(xbits, codes, scales, cols):
    xv = _torch_bf16(xbits)
    wv = _torch_e4m3(codes)
    K = codes.shape[1]
    out = []
    for m in range(xbits.shape[0]):
        row = []
        for n in cols:
            acc = Fraction(0)
            for kb in range(K // 128):
                part = Fraction(0)
                for k in range(kb * 128, kb * 128 + 128):
                    part += Fraction(float(xv[m, k])) * Fraction(float(wv[n, k]))
                acc += part * Fraction(float(scales[n // 128, kb]))
            row.append(acc)
        out.append(row)
    return out


def _check_against_exact(y64, exact, absdot, K):
    """Products are exact in binary64 (at most 36 significant bits), so a sequential
    sum of K of them is within K * 2^-53 * sum|x*w| of the exact value."""
    vals, bits = _all_finite("bf16")
    ov = _overflow_at("bf16")
    for m in range(len(exact)):
        for i, e in enumerate(exact[m]):
            bound = absdot[m][i] * K * Fraction(2) ** -53
            assert abs(Fraction(float(y64[m, i])) - e) <= bound, (m, i, float(y64[m, i]), float(e))
            # rounding of y64 to BF16 agrees with rounding of the exact sum (no boundary nearby)
            ref = oracle.bf16_rne(np.array([float(y64[m, i])]))[0]
            ex = _brute_round(float(e), vals, bits, 0x7F80, ov)
            assert int(ref) == ex, (m, i)


def pin_gemm_fp8_exact():
    rng = np.random.Generator(np.random.PCG64(23))
    M, N, K = 2, 256, 384
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    scales = rng.uniform(0.1, 4.0, size=(N // 128, K // 128)).astype(np.float32)
    xbits = synth.x_bf16(M, K, 24)
    cols = [0, 1, 77, 127, 128, 129, 200, 255]
    y64 = oracle.gemm_fp8(xbits, codes, scales, cols=cols)
    exact = _exact_fp8(xbits, codes, scales, cols)
    xv, wv = _torch_bf16(xbits), _torch_e4m3(codes)
    sfull = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    absdot = [[Fraction(float(np.abs(xv[m] * wv[n] * sfull[n]).sum())) * Fraction(101, 100) for n in cols]
              for m in range(M)]
    _check_against_exact(y64, exact, absdot, K)


def pin_gemm_lut3_exact():
    rng = np.random.Generator(np.random.PCG64(25))
    M, N, K = 2, 32, 384
    codes, qmap, g = synth.lut3_weights(N, K, 26)
    xbits = synth.x_f16(M, K, 27)
    cols = [0, 5, 16, 31]
    y64 = oracle.gemm_lut3(xbits, codes, qmap, g, cols=cols)
    xv = _numpy_f16(xbits)
    qv = _numpy_f16(qmap)
    gv = _numpy_f16(g)
    exact, absdot = [], []
    for m in range(M):
        row, ad = [], []
        for n in cols:
            acc = Fraction(0)
            tot = 0.0
            for k in range(K):
                w = float(np.float16(qv[codes[n, k]] * gv[n, k // 128]))
                acc += Fraction(float(xv[m, k])) * Fraction(w)
                tot += abs(float(xv[m, k]) * w)
            row.append(acc)
            ad.append(Fraction(tot) * Fraction(101, 100))
        exact.append(row)
        absdot.append(ad)
    _check_against_exact(y64, exact, absdot, K)
    del rng


def pin_integer_exact():
    rng = np.random.Generator(np.random.PCG64(28))
    M, N, K = 3, 128, 512
    wi = rng.integers(-8, 9, size=(N, K))
    xi = rng.integers(-2, 3, size=(M, K))
    codes = torch.from_numpy(wi.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = np.ones((N // 128, K // 128), dtype=np.float32)
    xbits = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y64 = oracle.gemm_fp8(xbits, codes, scales)
    assert np.array_equal(y64, (xi @ wi.T).astype(np.float64)), "FP8 integer case != int64 matmul"
    # LUT: map {-4..3}, unit group scales, FP16 activations in {-2..2}
    ci = rng.integers(0, 8, size=(N, K)).astype(np.uint8)
    qmap = np.arange(-4, 4).astype(np.float16).view(np.uint16)
    g = np.ones((N, K // 128), dtype=np.float16).view(np.uint16)
    xh = xi.astype(np.float16).view(np.uint16)
    y64 = oracle.gemm_lut3(xh, ci, qmap, g)
    assert np.array_equal(y64, (xi @ (ci.astype(np.int64) - 4).T).astype(np.float64)), "LUT integer case != int64 matmul"


def pin_closed_form():
    # x = +1 on row 0 and -1 on row 1; every code in row n is c_n; one scale per 128x128 block.
    N, K = 256, 256
    cvals = np.array([1.0, 1.5, 2.0, 3.5, 0.25, 7.0, 448.0, 2.0 ** -9], dtype=np.float32)
    cn = cvals[np.arange(N) % 8]
    codes = torch.from_numpy(np.repeat(cn[:, None], K, 1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    s = np.array([[0.5, 0.25], [2.0, 0.125]], dtype=np.float32)
    x = np.ones((2, K), dtype=np.float32)
    x[1] = -1
    xbits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y64 = oracle.gemm_fp8(xbits, codes, s)
    for n in range(N):
        want = 128.0 * float(cn[n]) * (float(s[n // 128, 0]) + float(s[n // 128, 1]))
        assert y64[0, n] == want and y64[1, n] == -want, (n, y64[0, n], want)


def pin_scale_linearity():
    N, K, M = 256, 384, 4
    codes, scales = synth.fp8_weights(N, K, 30)
    xbits = synth.x_bf16(M, K, 31)
    y = oracle.gemm_fp8(xbits, codes, scales)
    y2 = oracle.gemm_fp8(xbits, codes, scales * np.float32(2.0))
    y8 = oracle.gemm_fp8(xbits, codes, scales * np.float32(0.125))
    assert np.array_equal(y2, 2 * y) and np.array_equal(y8, y / 8), "FP8 scale linearity"
    c, q, g = synth.lut3_weights(64, K, 32)
    qf = q.view(np.float16).astype(np.float32)      # no FP16-subnormal products (doubling exact)
    q = np.where(np.abs(qf) < 0.02, np.copysign(0.02, qf), qf).astype(np.float16).view(np.uint16)
    xh = synth.x_f16(M, K, 33)
    g2 = (g.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    yl = oracle.gemm_lut3(xh, c, q, g)
    yl2 = oracle.gemm_lut3(xh, c, q, g2)
    assert np.array_equal(yl2, 2 * yl), "LUT scale linearity"


def pin_strides_rows_cols_threads():
    N, K = 256, 512
    codes, scales = synth.fp8_weights(N, K, 34)
    xb = synth.x_bf16(32, K, 35)
    xs = synth.x_bf16(32, K, 35, ld=K + 24)          # canary NaNs in the padding
    full = oracle.gemm_fp8(xb, codes, scales, nthreads=1)
    assert np.array_equal(oracle.gemm_fp8(xs, codes, scales, K=K, nthreads=5), full), "x stride / threads"
    halves = np.vstack([oracle.gemm_fp8(xb[:16], codes, scales), oracle.gemm_fp8(xb[16:], codes, scales)])
    assert np.array_equal(halves, full), "M=32 != two M=16 halves"
    cols = np.array([255, 3, 128, 7])
    assert np.array_equal(oracle.gemm_fp8(xb, codes, scales, cols=cols), full[:, cols]), "column subset"
    # strided weights: a wider code matrix whose padding is garbage
    wide = np.full((N, K + 128), 0x7F, dtype=np.uint8)
    wide[:, :K] = codes
    assert np.array_equal(oracle.gemm_fp8(xb, wide, scales, K=K), full), "weight stride"
    c, q, g = synth.lut3_weights(64, K, 36)
    xh = synth.x_f16(4, K, 37)
    xhs = synth.x_f16(4, K, 37, ld=K + 8)
    yl = oracle.gemm_lut3(xh, c, q, g, nthreads=1)
    assert np.array_equal(oracle.gemm_lut3(xhs, c, q, g, K=K, nthreads=3), yl), "LUT x stride / threads"


# -------------------------------------------------------------------- W8A8

def _e4m3_table():
    """The 254 finite E4M3FN values (library decode), their codes, sorted by value."""
    codes = np.arange(256, dtype=np.uint8)
    vals = _torch_e4m3(codes)
    keep = np.isfinite(vals)
    return vals[keep], codes[keep]


def _brute_e4m3(v: float, vals, codes) -> int:
    """Nearest finite E4M3 value by exhaustive search in exact rationals, ties to the even code;
    a negative value keeps its sign (rounds to -0 when it rounds to zero)."""
    fv = Fraction(v)
    best = None
    for val, code in zip(vals, codes):
        if val == 0 and (int(code) & 0x80) != (0x80 if math.copysign(1.0, v) < 0 else 0):
            continue
        d = abs(fv - Fraction(float(val)))
        key = (d, int(code) & 1)
        if best is None or key < best[0]:
            best = (key, int(code))
    return best[1]


def _e4m3_inputs(seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    vals, _ = _e4m3_table()
    pos = np.unique(vals[vals >= 0])
    v = list(pos) + list(-pos)
    for a, b in zip(pos[:-1], pos[1:]):            # ties and their float32 neighbours
        mid = np.float32((a + b) / 2)
        v += [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))]
    v += list(_rand_doubles(rng, 400, -12, 9).clip(-448, 448))
    v += [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -11]
    return np.array(v, dtype=np.float32)


def pin_e4m3_encode():
    v = _e4m3_inputs(40)
    got = oracle.e4m3_rne(v)
    # (1) torch's float32 -> float8_e4m3fn cast (round to nearest even)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want), "e4m3_rne != torch cast at %r" % v[np.argmax(got != want)]
    # (2) exhaustive nearest-value search in exact rationals
    vals, codes = _e4m3_table()
    for x, g in list(zip(v, got))[::3]:
        assert _brute_e4m3(float(x), vals, codes) == int(g), (float(x), hex(int(g)))


def _quant_fixture(seed: int, ld_pad: int = 0):
    """BF16 activations [5, 512 (+pad)]: random groups, an all-zero group, a group whose
    largest magnitude is negative, one with amax 448 (scale 1), tiny and huge groups."""
    M, K = 5, 512
    x = synth.normal_matrix(M, K, seed)
    x[1, 128:256] = 0.0
    x[2, 0:128] = np.abs(x[2, 0:128])
    x[2, 7] = -9.5
    x[3, 256:384] = np.clip(x[3, 256:384] * 40, -447, 447)
    x[3, 300] = 448.0
    x[4, 0:128] *= 1e-6
    x[4, 384:512] *= 3e4
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if ld_pad:
        wide = np.full((M, K + ld_pad), 0x7FC1, dtype=np.uint16)
        wide[:, :K] = bits
        return wide, K
    return bits, K


def pin_quantize_x():
    xb, K = _quant_fixture(41)
    codes, sc = oracle.quantize_x_fp8(xb)
    xv = _torch_bf16(xb).astype(np.float32)            # BF16 -> binary32 is exact
    for m in range(xb.shape[0]):
        for kb in range(K // 128):
            blk = xv[m, kb * 128:(kb + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            assert sc[m, kb] == s, (m, kb, sc[m, kb], s)
            q = np.clip(blk / s, np.float32(-448), np.float32(448)).astype(np.float32)   # numpy binary32 division
            want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[m, kb * 128:(kb + 1) * 128], want), (m, kb)
            if amax > 0:   # the largest magnitude lands on +-448 exactly
                i = int(np.argmax(np.abs(blk)))
                assert codes[m, kb * 128 + i] in (0x7E, 0xFE), (m, kb, hex(codes[m, kb * 128 + i]))
    assert sc[1, 1] == 1.0 and not codes[1, 128:256].any(), "all-zero group"
    assert sc[3, 2] == 1.0, "amax 448 gives scale 1"
    assert codes[2, 7] == 0xFE, "negative extreme"
    # the padding of a strided x is never read
    xs, _ = _quant_fixture(41, ld_pad=40)
    c2, s2 = oracle.quantize_x_fp8(xs, K=K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sc), "x stride"


def pin_quantize_x_nonfinite():
    """A K group holding +Inf, -Inf or NaN gets scale NaN and the E4M3 NaN
    code 0x7F everywhere (the reading for non-finite input); the row's other
    groups and the other rows quantise as without it."""
    xb, K = _quant_fixture(47)
    base_c, base_s = oracle.quantize_x_fp8(xb)
    bad = xb.copy()
    bad[0, 5] = 0x7F80        # +Inf in row 0, group 0
    bad[2, 300] = 0xFF80      # -Inf in row 2, group 2
    bad[4, 511] = 0x7FC1      # NaN in row 4, group 3
    c, s = oracle.quantize_x_fp8(bad)
    hit = {(0, 0), (2, 2), (4, 3)}
    for m in range(xb.shape[0]):
        for kb in range(K // 128):
            blk = slice(kb * 128, (kb + 1) * 128)
            if (m, kb) in hit:
                assert np.isnan(s[m, kb]) and np.all(c[m, blk] == 0x7F), (m, kb)
            else:
                assert s[m, kb] == base_s[m, kb] and np.array_equal(c[m, blk], base_c[m, blk]), (m, kb)
    # the product: every output of a row with such a group is NaN, the others are finite
    q = np.full((128, K), 0x38, dtype=np.uint8)       # E4M3 1.0
    y = oracle.gemm_w8a8(c, s, q, np.ones((1, K // 128), dtype=np.float32))
    assert np.all(np.isnan(y[[0, 2, 4]])) and np.all(np.isfinite(y[[1, 3]]))


def pin_gemm_w8a8_exact():
    rng = np.random.Generator(np.random.PCG64(42))
    M, N, K = 2, 256, 256
    xb = synth.x_bf16(M, K, 43)
    xq, sx = oracle.quantize_x_fp8(xb)
    q = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x31
    sw = rng.uniform(0.05, 3.0, size=(N // 128, K // 128)).astype(np.float32)
    cols = [0, 1, 100, 127, 128, 200, 255]
    wide = np.full((M, K + 64), 0x7F, dtype=np.uint8)            # NaN codes in the padding
    wide[:, :K] = xq
    y64 = oracle.gemm_w8a8(wide, sx, q, sw, K=K, cols=cols)
    xv, wv = _torch_e4m3(xq), _torch_e4m3(q)
    exact, absdot = [], []
    for m in range(M):
        row, ad = [], []
        for n in cols:
            acc, tot = Fraction(0), 0.0
            for k in range(K):
                a = Fraction(float(xv[m, k])) * Fraction(float(sx[m, k // 128]))
                b = Fraction(float(wv[n, k])) * Fraction(float(sw[n // 128, k // 128]))
                acc += a * b
                tot += abs(float(a * b))
            row.append(acc)
            ad.append(Fraction(tot) * Fraction(101, 100))
        exact.append(row)
        absdot.append(ad)
    _check_against_exact(y64, exact, absdot, K)


def pin_w8a8_integer_exact():
    """Groups holding 448 quantise with scale 1, so small integers pass through exactly."""
    rng = np.random.Generator(np.random.PCG64(44))
    M, N, K = 3, 128, 384
    xi = rng.integers(-6, 7, size=(M, K)).astype(np.int64)
    xi[:, ::128] = 448
    wi = rng.integers(-8, 9, size=(N, K))
    xb = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xq, sx = oracle.quantize_x_fp8(xb)
    assert np.all(sx == 1.0)
    q = torch.from_numpy(wi.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    y64 = oracle.gemm_w8a8(xq, sx, q, np.ones((1, K // 128), np.float32))
    assert np.array_equal(y64, (xi @ wi.T).astype(np.float64)), "W8A8 integer case != int64 matmul"


ALL_PINS = [
    pin_e4m3_all_codes, pin_e4m3_golden, pin_f16_decode_all, pin_bf16_decode_all, pin_16bit_golden,
    pin_f16_rne, pin_bf16_rne, pin_fp8_dequant, pin_lut_dequant, pin_lut_rejects_bad_code,
    pin_gemm_fp8_exact, pin_gemm_lut3_exact, pin_integer_exact, pin_closed_form,
    pin_scale_linearity, pin_strides_rows_cols_threads,
    pin_e4m3_encode, pin_quantize_x, pin_quantize_x_nonfinite, pin_gemm_w8a8_exact, pin_w8a8_integer_exact,
]
