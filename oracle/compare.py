"""Acceptance rule for a GEMM result against the binary64 oracle (test infrastructure).

The rule follows the numerics contract of the tensor-core decode tier in the atlas
"Module m16_tc" docs: section NUMERICS gives at most 2 BF16 ULP per element, and
section "THE ROUND-6 M=32 RED CELL WAS THE ORACLE" explains why a pure ULP budget
misgrades outputs that cancelled to almost nothing and calls for a mixed
absolute/relative criterion.  The absolute floor used here is
1e-3 * sqrt(K) * max|x| * max|w|.

Reading taken where the pages are silent:
* the two criteria are OR-ed: an element passes if it is within 2 BF16 ULP of
  bf16_rne(y64) **or** within the floor of y64;
* the ULP distance is measured on the BF16 ordinal (``bf16_ord``): non-negative
  patterns map to themselves, negative ones to -(bits & 0x7FFF), so +0 and -0 are
  both 0 and adjacent representable values differ by 1;
* an FP16 result (LUT path) is first rounded to BF16 (RNE) and then graded the same
  way; its FP16-ULP distance is reported alongside;
* a non-finite result fails unless the oracle's value is NaN too (NaN weights).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import bf16_rne, bf16_value, f16_rne, f16_value

MAX_ULP = 2
FLOOR_COEF = 1e-3
# Smallest FP16 normal.  Below it FP16's spacing is a fixed 2^-24, wider than
# 2 BF16 ULP of any value under 2^-16, so an FP16 output there can miss the
# ULP budget even when it is the correctly rounded result.
F16_MIN_NORMAL = 2.0 ** -14


def bf16_ord(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def f16_ord(bits) -> np.ndarray:
    return bf16_ord(bits)  # same sign-magnitude ordinal construction


def abs_floor(K: int, max_abs_x: float, max_abs_w: float) -> float:
    return FLOOR_COEF * math.sqrt(K) * float(max_abs_x) * float(max_abs_w)


@dataclasses.dataclass
class Receipt:
    n: int
    n_fail: int
    max_ulp: int
    n_over_budget: int          # elements beyond MAX_ULP (they may still pass via the floor)
    n_over_budget_resolvable: int  # of those, the ones the output format resolves to MAX_ULP
                                   # (FP16 output: |y64| at or above FP16's smallest normal)
    max_err_over_floor: float
    rel_rms: float
    sign_flips: int
    floor: float
    max_f16_ulp: int | None = None
    first_fail: tuple | None = None

    @property
    def ok(self) -> bool:
        return self.n_fail == 0

    def __str__(self) -> str:
        s = ("n=%d fail=%d max_ulp=%d over_2ulp=%d (resolvable %d) max_err/floor=%.3g rel_rms=%.3g "
             "sign_flips=%d floor=%.3g"
             % (self.n, self.n_fail, self.max_ulp, self.n_over_budget, self.n_over_budget_resolvable,
                self.max_err_over_floor, self.rel_rms, self.sign_flips, self.floor))
        if self.max_f16_ulp is not None:
            s += " max_f16_ulp=%d" % self.max_f16_ulp
        if self.first_fail is not None:
            s += " first_fail=%s" % (self.first_fail,)
        return s


def grade(y_bits: np.ndarray, y64: np.ndarray, floor: float, out_dtype: str = "bf16") -> Receipt:
    """Grade GPU output bits (uint16, BF16 or FP16) against y64 (float64), same shape."""
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    y64 = np.asarray(y64, dtype=np.float64)
    if y_bits.shape != y64.shape:
        raise ValueError("shape mismatch %s vs %s" % (y_bits.shape, y64.shape))
    if out_dtype == "bf16":
        g = bf16_value(y_bits)
        g_b = y_bits
        max_f16 = None
    elif out_dtype == "f16":
        g = f16_value(y_bits)
        g_b = bf16_rne(g)
        ref_h = f16_rne(y64)
        fin = np.isfinite(g) & np.isfinite(y64)
        max_f16 = int(np.abs(f16_ord(y_bits) - f16_ord(ref_h))[fin].max(initial=0))
    else:
        raise ValueError(out_dtype)
    ref_b = bf16_rne(y64)
    ulp = np.abs(bf16_ord(g_b) - bf16_ord(ref_b))
    both_nan = np.isnan(g) & np.isnan(y64)
    finite = np.isfinite(g)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - y64)
    ulp_ok = ulp <= MAX_ULP
    abs_ok = err <= floor
    ok = (finite & (ulp_ok | abs_ok)) | both_nan
    fin = finite & np.isfinite(y64)
    resolvable = fin & (np.abs(y64) >= F16_MIN_NORMAL) if out_dtype == "f16" else fin
    denom = math.sqrt(float(np.sum(y64[fin] ** 2))) if fin.any() else 0.0
    rel_rms = math.sqrt(float(np.sum((g[fin] - y64[fin]) ** 2))) / denom if denom > 0 else 0.0
    big = fin & (np.abs(y64) > floor)
    flips = int(np.sum(np.sign(g[big]) != np.sign(y64[big])))
    bad = np.argwhere(~ok)
    first = None
    if bad.size:
        idx = tuple(int(i) for i in bad[0])
        first = (idx, int(y_bits[idx]), float(g[idx]), float(y64[idx]))
    return Receipt(
        n=int(y64.size), n_fail=int((~ok).sum()),
        max_ulp=int(ulp[fin].max(initial=0)), n_over_budget=int((fin & ~ulp_ok).sum()),
        n_over_budget_resolvable=int((resolvable & ~ulp_ok).sum()),
        max_err_over_floor=float(err[fin].max(initial=0.0) / floor) if floor > 0 else float("inf"),
        rel_rms=rel_rms, sign_flips=flips, floor=floor, max_f16_ulp=max_f16, first_fail=first)
