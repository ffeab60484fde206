"""The no-allocation FP8 GEMM (wq_gemm_fp8_block_noalloc) through the C ABI:
its K-split partials live in the library's static device scratch instead of a
caller workspace.  Checked against the same call with a workspace
(wq_gemm_fp8_block): identical bits, on two calls in a row -- the FFN down
projection (its plan splits K into 4 parts, so the scratch holds the
partials) and then a smaller input (fewer rows, and a smaller shape with a
forced K split), each also graded against the oracle on sampled columns.
Shapes whose plan needs more scratch than the array holds are refused."""
import numpy as np
import pytest
import torch

import synth
import gpu_util as U

pytestmark = pytest.mark.gpu


def _both(packed, N, K, xbits):
    """(no-allocation output bits, with-workspace output bits) for the same call."""
    wq = U.wqmod()
    M = xbits.shape[0]
    x = U.t_u16(xbits, torch.bfloat16)
    y0 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=U.DEV)
    y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=U.DEV)
    wq.wq_gemm_fp8_block_noalloc(packed, N, K, x, y0, M)
    ws = wq.workspace(wq.WQ_FMT_FP8_BLOCK, N, K, U.DEV)
    wq.wq_gemm_fp8_block(packed, N, K, x, y1, M, ws)
    torch.cuda.synchronize()
    return U.bits_of(y0), U.bits_of(y1)


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    wq = U.wqmod()
    wq.wq_set_kparts(0)
    fmt, N, K, Ms, (codes, scales) = U.config_inputs("down")
    need = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, 32, N, K)
    assert 0 < need <= wq.wq_noalloc_scratch_bytes()          # the plan splits K: the scratch is used
    packed = U.pack_fp8(codes, scales)
    cols = U.sample_cols(N, 91)
    for M in (32, 8):                                         # the second call is smaller
        U.note("noalloc down N=%d K=%d M=%d" % (N, K, M))
        xb = synth.x_bf16(M, K, 1900 + M)
        y0, y1 = _both(packed, N, K, xb)
        assert np.array_equal(y0, y1), M
        U.check(U.grade_fp8(y0, xb, codes, scales, K, cols=cols), "noalloc M=%d" % M)
    # then a smaller shape with a forced 3-part split, after the larger call's partials
    N2, K2 = 640, 2560
    codes2, scales2 = synth.fp8_weights(N2, K2, 1950)
    packed2 = U.pack_fp8(codes2, scales2)
    wq.wq_set_kparts(3)
    try:
        for M in (16, 5):
            U.note("noalloc small N=%d K=%d M=%d kp=3" % (N2, K2, M))
            xb = synth.x_bf16(M, K2, 1960 + M)
            y0, y1 = _both(packed2, N2, K2, xb)
            assert np.array_equal(y0, y1), M
            U.check(U.grade_fp8(y0, xb, codes2, scales2, K2), "noalloc small M=%d" % M)
    finally:
        wq.wq_set_kparts(0)


def test_noalloc_refuses_a_plan_larger_than_the_scratch():
    wq = U.wqmod()
    N, K = 5120, 17408
    wq.wq_set_kparts(32)                                      # 32 x 32 x 5120 x 4 B > 4 MiB
    try:
        assert wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, 16, N, K) > wq.wq_noalloc_scratch_bytes()
        U.note("noalloc refuses kp=32")
        packed = torch.empty(wq.wq_fp8_block_packed_bytes(N, K), dtype=torch.uint8, device=U.DEV)
        x = torch.zeros((16, K), dtype=torch.bfloat16, device=U.DEV)
        y = torch.zeros((16, N), dtype=torch.bfloat16, device=U.DEV)
        with pytest.raises(wq.WqError) as e:
            wq.wq_gemm_fp8_block_noalloc(packed, N, K, x, y, 16)
        assert e.value.status == wq.WQ_ERR_SCRATCH
        torch.cuda.synchronize()
        assert not y.view(torch.int16).any()                   # nothing was queued
    finally:
        wq.wq_set_kparts(0)
