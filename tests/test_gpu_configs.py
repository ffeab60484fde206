"""Parity at the full workload sizes, in the launch configurations the
benchmark times (with the workspace the shape asks for, which splits K across
work-groups for the FFN down projection, and without one).  The oracle computes every column of the first and last 128 and 768
random columns in between (all M rows each); the comparison rule is the same
as at small sizes.  With WQ_RECEIPTS naming a file, each case appends its
receipt there as one JSON line."""
import json
import os

import numpy as np
import pytest

import synth
import gpu_util as U

pytestmark = pytest.mark.gpu

def _splits_k(fmt, M, N, K):
    """Whether the shape's plan on this device splits K across work-groups
    when given a workspace (the size query is host arithmetic plus the CU
    count; with no device it answers 0)."""
    try:
        wq = U.wqmod()
        wfmt = {"fp8": wq.WQ_FMT_FP8_BLOCK, "lut3": wq.WQ_FMT_LUT3, "lut3d": wq.WQ_FMT_LUT3_DENSE}[fmt]
        return wq.wq_gemm_workspace_bytes(wfmt, M, N, K) > 0
    except Exception:
        return False


# every config without a workspace; with the workspace the benchmark passes
# only where that changes the launch (K parts across work-groups)
CASES = [(name, M, ws) for name, (fmt, N, K, Ms) in synth.CONFIGS.items() for M in Ms
         for ws in (None, "auto") if ws is None or _splits_k(fmt, M, N, K)]
# the strict-order FP8 GEMV arm (explicit path; AUTO takes the MFMA tile) at
# the configs' M <= 4
CASES += [(name, M, "gemv") for name, (fmt, N, K, Ms) in synth.CONFIGS.items() if fmt == "fp8"
          for M in Ms if M <= 4]


@pytest.mark.parametrize("name,M,ws", CASES, ids=["%s-M%d-%s" % (n, m, w or "nows") for n, m, w in CASES])
def test_config_parity(name, M, ws):
    """ws None: no workspace (one K part); "auto": the workspace the shape asks
    for, as the benchmark passes; "gemv": the FP8 GEMV arm, no workspace."""
    fmt, N, K, Ms, data = U.config_inputs(name)
    wq = U.wqmod()
    wfmt = {"fp8": wq.WQ_FMT_FP8_BLOCK, "lut3": wq.WQ_FMT_LUT3, "lut3d": wq.WQ_FMT_LUT3_DENSE}[fmt]
    path = 1 if ws == "gemv" else 0
    ws = None if ws == "gemv" else ws
    assert not ws or wq.wq_gemm_workspace_bytes(wfmt, M, N, K) > 0
    U.note("config %s %s N=%d K=%d M=%d ws=%s path=%d" % (name, fmt, N, K, M, ws, path))
    cols = U.sample_cols(N, 7 + M)
    if fmt == "fp8":
        codes, scales = data
        xbits = synth.x_bf16(M, K, synth.SEEDS[name] + 100)
        packed = _packed(name, lambda: U.pack_fp8(codes, scales))
        y, _ = U.run_fp8(packed, N, K, xbits, ws=ws, path=path)
        r = U.grade_fp8(y, xbits, codes, scales, K, cols=cols)
    else:
        codes, qmap, g = data
        xbits = synth.x_f16(M, K, synth.SEEDS[name] + 100)
        dense = fmt == "lut3d"
        packed = _packed(name, lambda: U.pack_lut3(codes, qmap, g, dense=dense))
        y, _ = U.run_lut3(packed, N, K, xbits, ws=ws, dense=dense)
        r = U.grade_lut3(y, xbits, codes, qmap, g, K, cols=cols)
    U.note("  %s" % r)
    if os.environ.get("WQ_RECEIPTS"):   # a file to append the receipt to (one JSON line per case)
        with open(os.environ["WQ_RECEIPTS"], "a") as f:
            f.write(json.dumps({"config": name, "M": M, "workspace": ws, "path": "gemv" if path else "auto",
                                "n": r.n, "max_ulp": r.max_ulp, "over_2ulp": r.n_over_budget,
                                "over_2ulp_resolvable": r.n_over_budget_resolvable, "rel_rms": r.rel_rms,
                                "sign_flips": r.sign_flips, "max_err_over_floor": r.max_err_over_floor,
                                "floor": r.floor, "max_f16_ulp": r.max_f16_ulp}) + "\n")
    U.check(r, out_dtype="bf16" if fmt == "fp8" else "f16")


_PACKED = {}


def _packed(name, make):
    if name not in _PACKED:
        _PACKED.clear()            # keep one packed matrix resident at a time
        _PACKED[name] = make()
    return _PACKED[name]
