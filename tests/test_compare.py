"""The acceptance rule (oracle/compare.py) grades what it should: exact and
near results pass, results beyond 2 BF16 ULP fail unless within the absolute
floor (the cancellation case of the atlas m16_tc docs' M=32 red cell), and
non-finite results fail unless the reference is NaN too."""
import numpy as np

import oracle
from oracle import compare as C


def bits(v):
    return oracle.bf16_rne(np.asarray(v, dtype=np.float64))


def step(b, k):
    """Move a BF16 pattern k ordinal steps (positive = towards +inf)."""
    o = C.bf16_ord(np.array([b]))[0] + k
    return np.uint16(o if o >= 0 else 0x8000 | (-o))


def test_ord_is_monotone_and_signed_zero_agnostic():
    v = np.array([-3.0, -1.0, -2.0 ** -130, -0.0, 0.0, 2.0 ** -130, 1.0, 3.0])
    o = C.bf16_ord(bits(v))
    assert list(o) == sorted(o)
    assert o[3] == o[4] == 0


def test_exact_and_two_ulp_pass_three_fail():
    y64 = np.array([[1.5, -37.25, 1000.0]])
    b = bits(y64)
    assert C.grade(b, y64, floor=1e-9).ok
    plus2 = np.array([[step(x, 2) for x in b[0]]])
    assert C.grade(plus2, y64, floor=1e-9).ok
    plus3 = np.array([[step(x, -3) for x in b[0]]])
    r = C.grade(plus3, y64, floor=1e-9)
    assert r.n_fail == 3 and r.max_ulp == 3


def test_cancellation_passes_through_the_floor():
    # an output that cancelled to ~1e-6 of the matrix scale: hundreds of ULP off, tiny absolute error
    y64 = np.array([[5.7e-6, 39.1]])
    g = np.array([[bits(5.7e-6 + 3e-6)[0], bits(39.1)[0]]])
    r = C.grade(g, y64, floor=C.abs_floor(5120, 4.0, 0.1))
    assert r.ok and r.max_ulp > 2 and r.n_over_budget == 1
    r2 = C.grade(g, y64, floor=1e-7)
    assert not r2.ok


def test_non_finite():
    y64 = np.array([[1.0, float("nan")]])
    nan = np.uint16(0x7FC0)
    assert not C.grade(np.array([[nan, nan]]), y64, floor=1.0).ok         # NaN where a number is due
    assert C.grade(np.array([[bits(1.0)[0], nan]]), y64, floor=1.0).ok   # NaN where NaN is due
    inf = np.uint16(0x7F80)
    assert not C.grade(np.array([[inf, nan]]), y64, floor=1e30).ok


def test_f16_output_graded_after_bf16_rounding():
    y64 = np.array([[0.333251953125, -2.0]])   # exactly representable in FP16
    h = oracle.f16_rne(y64)
    r = C.grade(h, y64, floor=1e-9, out_dtype="f16")
    assert r.ok and r.max_f16_ulp == 0
    h2 = h.copy()
    h2[0, 0] += 40                              # 40 FP16 ULP = 5 BF16 ULP
    r2 = C.grade(h2, y64, floor=1e-9, out_dtype="f16")
    assert not r2.ok and r2.max_f16_ulp == 40


def test_sign_flips_counted_only_above_floor():
    y64 = np.array([[2.0, 1e-8]])
    g = bits(np.array([[-2.0, -1e-8]]))
    r = C.grade(g, y64, floor=1e-6)
    assert r.sign_flips == 1
