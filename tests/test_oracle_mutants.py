"""Mutation tests of the oracle's pins (CPU only).

Each case plants one plausible mistake in a private copy of oracle/oracle.c
(a dropped term, a wrong sign, bias, index, stride or rounding rule, a transposed
output), compiles it with gcc into a temporary library and runs the pin suite
against it.  The case passes only if at least one pin fails -- i.e. the pins
would have caught that mistake in the real oracle.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (id, text to find, replacement, which occurrence (None = all))
MUTANTS = [
    ("e4m3_bias", "e - 7 - 3", "e - 8 - 3", None),
    ("e4m3_subnormal_scale", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);", None),
    ("e4m3_sign_dropped", "return s ? -v : v;", "return v;", 0),
    ("e4m3_nan_missing", "if (e == 15 && m == 7)\n        return NAN;", "if (0)\n        return NAN;", None),
    ("f16_subnormal_scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);", None),
    ("bf16_bias", "e - 127 - 7", "e - 126 - 7", None),
    ("rne_truncates", "double q = nearbyint(ldexp(a, (p - 1) - e));", "double q = floor(ldexp(a, (p - 1) - e));", None),
    ("rne_ties_away", "double q = nearbyint(ldexp(a, (p - 1) - e));", "double q = round(ldexp(a, (p - 1) - e));", None),
    ("rne_subnormal_truncates", "double q = nearbyint(ldexp(a, (p - 1) - emin));", "double q = floor(ldexp(a, (p - 1) - emin));", None),
    ("rne_exponent_bias", "uint32_t field = (uint32_t)(e + bias);", "uint32_t field = (uint32_t)(e + bias + 1);", None),
    ("rne_no_overflow", "if (e > emax) {", "if (e > emax + 1) {", None),
    ("fp8_scale_kblock_size", "(n / WQO_BLOCK) * kb + k / WQO_BLOCK", "(n / WQO_BLOCK) * kb + k / 256", None),
    ("fp8_scale_kblock_reversed", "(n / WQO_BLOCK) * kb + k / WQO_BLOCK", "(n / WQO_BLOCK) * kb + (kb - 1 - k / WQO_BLOCK)", None),
    ("fp8_scale_row_ignored", "(n / WQO_BLOCK) * kb + k / WQO_BLOCK", "k / WQO_BLOCK", None),
    ("lut_no_fp16_rounding", "w[k] = wqo_f16_value(wqo_f16_rne(p));", "w[k] = p;", None),
    ("lut_qmap_reversed", "qmap[code]", "qmap[7 - code]", None),
    ("lut_group_index", "g[n * kg + k / WQO_BLOCK]", "g[n * kg + (k / WQO_BLOCK + 1) % kg]", None),
    ("gemm_drops_last_k", "for (int64_t k = 0; k < j->K; ++k)\n                acc +=", "for (int64_t k = 0; k < j->K - 1; ++k)\n                acc +=", None),
    ("gemm_drops_first_k", "for (int64_t k = 0; k < j->K; ++k)\n                acc +=", "for (int64_t k = 1; k < j->K; ++k)\n                acc +=", None),
    ("gemm_subtracts", "acc += xr[k] * wrow[k];", "acc -= xr[k] * wrow[k];", None),
    ("gemm_row_zero_only", "const double* xr = j->x + m * j->K;", "const double* xr = j->x;", None),
    ("gemm_output_transposed", "j->y[m * j->ncols + ci] = acc;", "j->y[ci * j->M + m] = acc;", None),
    ("x_stride_ignored", "x_bits[m * ldx + k]", "x_bits[m * K + k]", None),
    ("e4m3enc_ties_away", "double q = nearbyint(ldexp(a, 3 - E));", "double q = round(ldexp(a, 3 - E));", None),
    ("e4m3enc_truncates", "double q = nearbyint(ldexp(a, 3 - E));", "double q = floor(ldexp(a, 3 - E));", None),
    ("e4m3enc_sub_truncates", "double m = nearbyint(ldexp(a, 9));", "double m = floor(ldexp(a, 9));", None),
    ("e4m3enc_sub_threshold", "if (a < ldexp(1.0, -6)) {", "if (a < ldexp(1.0, -7)) {", None),
    ("e4m3enc_bias", "((E + 7) << 3)", "((E + 8) << 3)", None),
    ("e4m3enc_carry_lost", "q = 8.0;\n        E += 1;", "q = 15.0;", None),
    ("e4m3enc_sign_dropped", "uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = 0x00;", None),
    ("quant_scale_const", "amax / 448.0f", "amax / 447.0f", None),
    ("quant_zero_group", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 448.0f : 0.5f", None),
    ("quant_amax_signed", "float a = fabsf((float)wqo_bf16_value(xr[i]));", "float a = (float)wqo_bf16_value(xr[i]);", None),
    ("quant_x_stride", "x_bf16 + m * ldx + kb * WQO_BLOCK", "x_bf16 + m * K + kb * WQO_BLOCK", None),
    ("quant_multiplies", "(float)wqo_bf16_value(xr[i]) / s;", "(float)wqo_bf16_value(xr[i]) * (1.0f / s);", None),
    ("w8a8_sx_group", "sx[m * kb_n + k / WQO_BLOCK]", "sx[m * kb_n]", None),
    ("w8a8_sx_row", "sx[m * kb_n + k / WQO_BLOCK]", "sx[k / WQO_BLOCK]", None),
    ("w8a8_x_stride", "xq[m * ldxq + k]", "xq[m * K + k]", None),
    ("quant_nonfinite_ignored", "if (!isfinite(a)) nonfinite = 1;", "if (0) nonfinite = 1;", None),
    ("quant_nonfinite_scale_one", "scales[m * kb_n + kb] = NAN;", "scales[m * kb_n + kb] = 1.0f;", None),
]


def _mutate(text, find, repl, which):
    n = text.count(find)
    assert n >= 1, "mutation anchor not found: %r" % find
    if which is None:
        return text.replace(find, repl)
    parts = text.split(find)
    return find.join(parts[: which + 1]) + repl + find.join(parts[which + 1:])


@pytest.mark.parametrize("mid,find,repl,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, find, repl, which):
    with open(SRC) as f:
        text = f.read()
    src = tmp_path / ("%s.c" % mid)
    src.write_text(_mutate(text, find, repl, which))
    lib = tmp_path / ("lib%s.so" % mid)
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(lib), "-lm"])
    caught = None
    with oracle.using(str(lib)):
        for pin in P.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError) as e:
                caught = (pin.__name__, str(e)[:120])
                break
    assert caught is not None, "mutant %s survived every pin" % mid
