"""The acceptance rule (oracle/compare.py) grades what it should: exact and
near results pass, results beyond 2 BF16 ULP fail unless within the absolute
floor (the cancellation case of the atlas m16_tc docs' M=32 red cell), and
non-finite results fail unless the reference is NaN too.

The floor is pinned to values the contract fixes (1e-3 * sqrt(K) * max|x| *
max|w| evaluated by hand at chosen points, written out as numbers), and the
element rule to the boundary on both sides of the floor and of the 2-ULP
budget.  Every pin is a function of the comparator module, so the mutation
test at the bottom can run the same pins against deliberately broken copies
of compare.py and require each copy to fail one of them.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest

import oracle
from oracle import compare as C_REAL

SRC = os.path.join(os.path.dirname(oracle.__file__), "compare.py")


def bits(v):
    return oracle.bf16_rne(np.asarray(v, dtype=np.float64))


def step(C, b, k):
    """Move a BF16 pattern k ordinal steps (positive = towards +inf)."""
    o = C.bf16_ord(np.array([b]))[0] + k
    return np.uint16(o if o >= 0 else 0x8000 | (-o))


# ---------------------------------------------------------------- pins

def pin_floor_values(C):
    """1e-3 * sqrt(K) * max|x| * max|w| at points where it is a short decimal."""
    cases = [  # K, max|x|, max|w|, floor
        (10000, 2.0, 0.5, 0.1),
        (1, 1.0, 1.0, 0.001),
        (16, 1.0, 1.0, 0.004),
        (256, 3.0, 0.25, 0.012),
        (4, 0.5, 8.0, 0.008),
        (1024, 1.0, 1.0, 0.032),
    ]
    for K, mx, mw, want in cases:
        got = C.abs_floor(K, mx, mw)
        assert abs(got - want) <= 1e-15 * want, (K, mx, mw, got, want)
    # K = 5120, max|x| = 4.688, max|w| = 0.1177 (the FFN gate/up magnitudes):
    # sqrt(5120) = 71.5541753, x 4.688 = 335.445974, x 0.1177 = 39.4819911, x 1e-3
    got = C.abs_floor(5120, 4.688, 0.1177)
    assert abs(got - 0.0394819911) < 1e-10, got


def pin_floor_boundary(C):
    """An element 10 ULP away passes just inside the floor and fails just outside."""
    y = 1.0
    far = step(C, bits(y)[0], 10)               # 10 BF16 ULP above 1.0: 1 + 10 * 2^-7
    err = float(oracle.bf16_value(np.array([far]))[0]) - y
    y64 = np.array([[y]])
    g = np.array([[far]])
    assert C.grade(g, y64, floor=err / 0.99).ok
    assert not C.grade(g, y64, floor=err / 1.01).ok
    assert C.grade(g, y64, floor=err).ok        # the floor itself is inside


def pin_exact_and_two_ulp_pass_three_fail(C):
    y64 = np.array([[1.5, -37.25, 1000.0]])
    b = bits(y64)
    assert C.grade(b, y64, floor=1e-9).ok
    for k in (1, 2, -1, -2):
        moved = np.array([[step(C, x, k) for x in b[0]]])
        r = C.grade(moved, y64, floor=1e-9)
        assert r.ok and r.max_ulp == abs(k) and r.n_over_budget == 0
    plus3 = np.array([[step(C, x, -3) for x in b[0]]])
    r = C.grade(plus3, y64, floor=1e-9)
    assert r.n_fail == 3 and r.max_ulp == 3 and r.n_over_budget == 3


def pin_criteria_are_or_ed(C):
    """Within 2 ULP but beyond the floor passes; beyond 2 ULP but within the
    floor passes; beyond both fails."""
    y64 = np.array([[100.0]])
    two = np.array([[step(C, bits(100.0)[0], 2)]])     # 2 ULP at 100 = 1.0 absolute
    assert C.grade(two, y64, floor=1e-6).ok
    five = np.array([[step(C, bits(100.0)[0], 5)]])    # 2.5 absolute
    assert C.grade(five, y64, floor=3.0).ok
    assert not C.grade(five, y64, floor=2.0).ok


def pin_ord_is_monotone_and_signed_zero_agnostic(C):
    v = np.array([-3.0, -1.0, -2.0 ** -130, -0.0, 0.0, 2.0 ** -130, 1.0, 3.0])
    o = C.bf16_ord(bits(v))
    assert list(o) == sorted(o) and len(set(o[[0, 1, 2, 5, 6, 7]])) == 6
    assert o[3] == o[4] == 0
    # across zero: the smallest negative and positive subnormals are 2 apart
    assert C.bf16_ord(np.array([0x0001]))[0] - C.bf16_ord(np.array([0x8001]))[0] == 2
    # ULP distance across the sign: +min and -min subnormal are within 2 ULP
    y64 = np.array([[2.0 ** -133]])
    assert C.grade(np.array([[np.uint16(0x8001)]]), y64, floor=0.0).ok
    assert not C.grade(np.array([[np.uint16(0x8002)]]), y64, floor=0.0).ok


def pin_cancellation_passes_through_the_floor(C):
    # an output that cancelled to ~1e-6 of the matrix scale: hundreds of ULP off, tiny absolute error
    y64 = np.array([[5.7e-6, 39.1]])
    g = np.array([[bits(5.7e-6 + 3e-6)[0], bits(39.1)[0]]])
    r = C.grade(g, y64, floor=C.abs_floor(5120, 4.0, 0.1))
    assert r.ok and r.max_ulp > 2 and r.n_over_budget == 1
    r2 = C.grade(g, y64, floor=1e-7)
    assert not r2.ok


def pin_non_finite(C):
    y64 = np.array([[1.0, float("nan")]])
    nan = np.uint16(0x7FC0)
    assert not C.grade(np.array([[nan, nan]]), y64, floor=1.0).ok         # NaN where a number is due
    assert C.grade(np.array([[bits(1.0)[0], nan]]), y64, floor=1.0).ok   # NaN where NaN is due
    inf = np.uint16(0x7F80)
    assert not C.grade(np.array([[inf, nan]]), y64, floor=1e30).ok
    assert not C.grade(np.array([[inf]]), np.array([[float("inf")]]), floor=1e30).ok


def pin_f16_output_graded_after_bf16_rounding(C):
    y64 = np.array([[0.333251953125, -2.0]])   # exactly representable in FP16
    h = oracle.f16_rne(y64)
    r = C.grade(h, y64, floor=1e-9, out_dtype="f16")
    assert r.ok and r.max_f16_ulp == 0
    h2 = h.copy()
    h2[0, 0] += 40                              # 40 FP16 ULP = 5 BF16 ULP
    r2 = C.grade(h2, y64, floor=1e-9, out_dtype="f16")
    assert not r2.ok and r2.max_f16_ulp == 40
    h3 = h.copy()
    h3[0, 0] += 8                               # 8 FP16 ULP = 1 BF16 ULP
    r3 = C.grade(h3, y64, floor=1e-9, out_dtype="f16")
    assert r3.ok and r3.max_ulp == 1


def pin_f16_resolvable_budget(C):
    """An FP16 output below FP16's smallest normal (2^-14) is counted over
    the budget but not as resolvable; at or above it, both.  At 2^-18 one
    FP16 step (2^-24) is 2 BF16 ULP, so 3 FP16 steps are 6 BF16 ULP."""
    y64 = np.array([[2.0 ** -18, 1.0]])
    h = oracle.f16_rne(y64)
    h[0, 0] += 3                                # 3 FP16 steps of 2^-24 above 2^-18
    h[0, 1] += 40                               # 40 FP16 ULP at 1.0 = 5 BF16 ULP
    r = C.grade(h, y64, floor=1.0, out_dtype="f16")
    assert r.ok and r.max_ulp == 6
    assert r.n_over_budget == 2 and r.n_over_budget_resolvable == 1
    rb = C.grade(bits(np.array([[1.0 + 5 * 2 ** -7, 2.0 ** -18 * (1 + 5 * 2 ** -7)]])),
                 np.array([[1.0, 2.0 ** -18]]), floor=1.0)
    assert rb.n_over_budget == rb.n_over_budget_resolvable == 2      # BF16 output: every element
    y_edge = np.array([[2.0 ** -14]])           # the smallest normal itself is resolvable
    he = oracle.f16_rne(y_edge) + 40
    re_ = C.grade(he, y_edge, floor=1.0, out_dtype="f16")
    assert re_.n_over_budget_resolvable == 1


def pin_sign_flips_counted_only_above_floor(C):
    y64 = np.array([[2.0, 1e-8]])
    g = bits(np.array([[-2.0, -1e-8]]))
    r = C.grade(g, y64, floor=1e-6)
    assert r.sign_flips == 1


def pin_rel_rms(C):
    """rel_rms = ||g - y64||_2 / ||y64||_2 over finite elements."""
    y64 = np.array([[3.0, 4.0]])                # norm 5
    g = bits(np.array([[3.0, 4.0 + 2 ** -5]]))  # 4 + 1/32 is a BF16 value (1 ULP at 4)
    r = C.grade(g, y64, floor=1.0)
    assert abs(r.rel_rms - (2 ** -5) / 5.0) < 1e-15
    assert r.n == 2 and r.n_fail == 0


COMPARE_PINS = [pin_floor_values, pin_floor_boundary, pin_exact_and_two_ulp_pass_three_fail,
                pin_criteria_are_or_ed, pin_ord_is_monotone_and_signed_zero_agnostic,
                pin_cancellation_passes_through_the_floor, pin_non_finite,
                pin_f16_output_graded_after_bf16_rounding, pin_f16_resolvable_budget,
                pin_sign_flips_counted_only_above_floor, pin_rel_rms]


@pytest.mark.parametrize("pin", COMPARE_PINS, ids=[p.__name__ for p in COMPARE_PINS])
def test_pin_holds(pin):
    pin(C_REAL)


# ---------------------------------------------------------------- mutants

# (id, text to find, replacement): one plausible mistake each
MUTANTS = [
    ("floor_no_sqrt", "math.sqrt(K)", "K", None),
    ("floor_coef_x10", "FLOOR_COEF = 1e-3", "FLOOR_COEF = 1e-2", None),
    ("floor_coef_div10", "FLOOR_COEF = 1e-3", "FLOOR_COEF = 1e-4", None),
    ("floor_drops_w", "* float(max_abs_x) * float(max_abs_w)", "* float(max_abs_x)", None),
    ("floor_sqrt_of_k_plus_1", "math.sqrt(K)", "math.sqrt(K + 1)", None),
    ("criteria_and", "(finite & (ulp_ok | abs_ok))", "(finite & (ulp_ok & abs_ok))", None),
    ("max_ulp_3", "MAX_ULP = 2", "MAX_ULP = 3", None),
    ("max_ulp_1", "MAX_ULP = 2", "MAX_ULP = 1", None),
    ("ulp_strict", "ulp_ok = ulp <= MAX_ULP", "ulp_ok = ulp < MAX_ULP", None),
    ("floor_strict", "abs_ok = err <= floor", "abs_ok = err < floor", None),
    ("ord_no_negation", "np.where(b & 0x8000, -(b & 0x7FFF), b)", "np.where(b & 0x8000, (b & 0x7FFF), b)", None),
    ("ord_raw_bits", "return np.where(b & 0x8000, -(b & 0x7FFF), b)", "return b", None),
    ("nan_always_ok", "ok = (finite & (ulp_ok | abs_ok)) | both_nan", "ok = (finite & (ulp_ok | abs_ok)) | np.isnan(g)", None),
    ("inf_allowed", "ok = (finite & (ulp_ok | abs_ok)) | both_nan", "ok = (ulp_ok | abs_ok) | both_nan", None),
    ("f16_graded_raw", "g_b = bf16_rne(g)", "g_b = y_bits", None),
    ("rel_rms_no_sqrt", "rel_rms = math.sqrt(float(np.sum((g[fin] - y64[fin]) ** 2))) / denom",
     "rel_rms = float(np.sum((g[fin] - y64[fin]) ** 2)) / denom", None),
    ("flips_everywhere", "big = fin & (np.abs(y64) > floor)", "big = fin", None),
    ("over_budget_counts_fails", "n_over_budget=int((fin & ~ulp_ok).sum())", "n_over_budget=int((~ok).sum())", None),
    ("resolvable_everything", "resolvable = fin & (np.abs(y64) >= F16_MIN_NORMAL) if", "resolvable = fin if", None),
    ("resolvable_threshold_bf16", "F16_MIN_NORMAL = 2.0 ** -14", "F16_MIN_NORMAL = 2.0 ** -126", None),
    ("resolvable_threshold_high", "F16_MIN_NORMAL = 2.0 ** -14", "F16_MIN_NORMAL = 2.0 ** -13", None),
    ("resolvable_for_bf16_too", 'if out_dtype == "f16" else fin', "", None),
]


def _load_mutant(text: str, tag: str):
    name = "oracle._compare_%s" % tag
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[name] = mod            # dataclasses look their module up while the class is built
    try:
        exec(compile(text, "compare_%s.py" % tag, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def test_unmutated_copy_passes_every_pin():
    with open(SRC) as f:
        mod = _load_mutant(f.read(), "copy")
    for pin in COMPARE_PINS:
        pin(mod)


@pytest.mark.parametrize("mid,find,repl,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_compare_mutant_is_caught(mid, find, repl, which):
    with open(SRC) as f:
        text = f.read()
    assert text.count(find) >= 1, "mutation anchor not found: %r" % find
    mod = _load_mutant(text.replace(find, repl), mid)
    caught = None
    for pin in COMPARE_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, TypeError) as e:
            caught = (pin.__name__, str(e)[:120])
            break
    assert caught is not None, "compare.py mutant %s survived every pin" % mid
