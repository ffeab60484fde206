"""The C-ABI library loads, exports every function include/wq.h declares, and
validates arguments on the host before any device work (CPU-only; no GPU is
touched except the 'no device' path, which must fail cleanly)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")

wq = pytest.importorskip("weight_only_quantized_fp8_amd.wq")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("wq_pack_fp8_block", "wq_gemm_fp8_block", "wq_pack_lut3", "wq_gemm_lut3",
                     "wq_gemm_workspace_bytes", "wq_unpack_fp8_block", "wq_unpack_lut3",
                     "wq_fp8_block_packed_bytes", "wq_lut3_packed_bytes", "wq_status_str",
                     "wq_packed_format_version"):
        assert required in names


PAGES = ("atlas docs", "FLUTE PR", "arc PR", "strata PR")


def test_every_declaration_cites_its_source():
    """Each declared call has its own comment directly above it, and the
    comment names the passage that defines the operation ("Source:" and a
    page); a call that exists for callers rather than for a passage says so
    ("Callers:")."""
    text = open(HEADER).read()
    decl = re.compile(r"^(?:const char\*|int|wq_status|size_t)\s+(wq_[a-z0-9_]+)\(", re.M)
    found = 0
    for m in decl.finditer(text):
        found += 1
        before = text[:m.start()].rstrip()
        assert before.endswith("*/"), "%s has no comment directly above it" % m.group(1)
        comment = before[before.rfind("/*"):]
        if "Callers:" in comment:
            continue
        assert "Source:" in comment, "%s: no Source: line" % m.group(1)
        cite = " ".join(comment[comment.find("Source:"):].split())
        assert any(p in cite for p in PAGES), "%s: the Source line names no page" % m.group(1)
    assert found == len(declared_functions())


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(wq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_wraps_every_declared_symbol():
    missing = [n for n in declared_functions() if not callable(getattr(wq, n, None))]
    assert not missing, missing


def test_status_strings():
    for s in range(10):
        assert wq.wq_status_str(s).startswith("WQ_")
    assert wq.wq_status_str(1234) == "WQ_ERR_UNKNOWN"


def test_workspace_bytes_without_a_device_are_zero():
    """The workspace size depends on the device's plan; with no gfx950 device
    current (this host) the query returns 0, and so it does for bad shapes."""
    for fmt, N, K in ((0, 17408, 5120), (0, 5120, 17408), (0, 256, 512), (1, 28672, 8192), (1, 48, 256),
                      (2, 28672, 8192), (0, 100, 512), (1, 48, 100), (7, 256, 512)):
        assert wq.wq_gemm_workspace_bytes(fmt, 16, N, K) == 0


def test_kparts_hook_validates():
    with pytest.raises(wq.WqError):
        wq.wq_set_kparts(-1)
    with pytest.raises(wq.WqError):
        wq.wq_set_kparts(33)
    for kp in (0, 1, 32, 0):
        wq.wq_set_kparts(kp)


def test_w8a8_stages_hook_validates():
    for bad in (-1, 1, 3, 5, 8):
        with pytest.raises(wq.WqError):
            wq.wq_set_w8a8_stages(bad)
    for ns in (0, 2, 4, 0):
        wq.wq_set_w8a8_stages(ns)


def test_sizes_are_host_arithmetic():
    assert wq.wq_packed_format_version() == 3
    assert wq.wq_fp8_block_packed_bytes(17408, 5120) == 17408 * 5120 + 4 * 136 * 40
    assert wq.wq_lut3_packed_bytes(28672, 8192) == 28672 * 8192 // 2 + 2 * 28672 * 64 + 32
    assert wq.wq_fp8_block_packed_bytes(100, 128) == 0      # N not a multiple of 128
    assert wq.wq_fp8_block_packed_bytes(128, 100) == 0
    assert wq.wq_lut3_packed_bytes(24, 128) == 0           # N not a multiple of 16
    assert wq.wq_lut3_packed_bytes(48, 256) == 48 * 128 + 3 * 256 + 32   # K blocks padded to 8
    # dense: 3 bits a code, the same scales, map and status word
    assert wq.wq_lut3_dense_packed_bytes(28672, 8192) == 28672 * 8192 * 3 // 8 + 2 * 28672 * 64 + 32
    assert wq.wq_lut3_dense_packed_bytes(48, 256) == 48 * 96 + 3 * 256 + 32
    assert wq.wq_lut3_dense_packed_bytes(24, 128) == 0
    assert wq.wq_lut3_dense_packed_bytes(32, 100) == 0


L = wq.lib
P = 1 << 20          # a 16-byte-aligned fake address; validation fails before it is used
BIG = 1 << 30


@pytest.mark.parametrize("args,expect", [
    # (packed, N, K, x, ldx, y, ldy, M, ws, ws_bytes)
    ((None, 256, 512, P, 512, P, 256, 1, P, BIG), 1),
    ((P, 256, 512, None, 512, P, 256, 1, P, BIG), 1),
    ((P, 256, 512, P, 512, None, 256, 1, P, BIG), 1),
    ((P, 256, 512, P, 512, P, 256, 33, P, BIG), 2),
    ((P, 256, 512, P, 512, P, 256, -1, P, BIG), 2),
    ((P, 200, 512, P, 512, P, 256, 1, P, BIG), 2),
    ((P, 256, 500, P, 512, P, 256, 1, P, BIG), 2),
    ((P, 0, 512, P, 512, P, 256, 1, P, BIG), 2),
    ((P, 256, 512, P, 511, P, 256, 1, P, BIG), 3),
    ((P, 256, 512, P, 512, P, 255, 1, P, BIG), 3),
    ((P, 256, 512, P, 516, P, 256, 1, P, BIG), 8),
    ((P + 8, 256, 512, P, 512, P, 256, 1, P, BIG), 8),
    ((P, 256, 512, P + 2, 512, P, 256, 1, P, BIG), 8),
    ((P, 256, 512, P, 512, P + 1, 256, 1, P, BIG), 8),
])
def test_fp8_gemm_validation(args, expect):
    assert L.wq_gemm_fp8_block(*args, None) == expect


def test_size_limits():
    # N, K at most 2^24 and N*K at most 2^35: the kernels' 32-bit buffer offsets
    assert wq.wq_fp8_block_packed_bytes(1 << 24, 128) > 0
    assert wq.wq_fp8_block_packed_bytes((1 << 24) + 128, 128) == 0
    assert wq.wq_fp8_block_packed_bytes(128, (1 << 24) + 128) == 0
    assert wq.wq_fp8_block_packed_bytes(1 << 24, 1 << 11) > 0          # 2^35 codes
    assert wq.wq_fp8_block_packed_bytes(1 << 24, (1 << 11) + 128) == 0
    assert wq.wq_lut3_packed_bytes(1 << 24, (1 << 11) + 128) == 0
    assert L.wq_gemm_fp8_block(P, (1 << 24) + 128, 512, P, 512, P, 1 << 25, 1, P, BIG, None) == 2
    assert L.wq_gemm_lut3(P, 1 << 24, 1 << 12, P, 1 << 12, P, 1 << 24, 1, P, BIG, None) == 2
    # activation span ((min(M, 32) - 1) * ldx + K) * 2 bytes under 4 GiB
    ld = 1 << 27
    assert L.wq_gemm_fp8_block(P, 256, 512, P, ld, P, 256, 32, P, BIG, None) == 3   # 31 * 2^28 + 1 KiB
    assert L.wq_gemm_lut3(P, 48, 512, P, ld, P, 48, 17, P, BIG, None) == 3      # 16 * 2^28 + 1 KiB
    assert L.wq_gemm_fp8_block(P, 256, 512, P, 1 << 60, P, 256, 1, P, BIG, None) == 3


def test_m_zero_is_a_no_op():
    # M == 0 queues nothing and returns WQ_OK before looking at the pointers
    assert L.wq_gemm_fp8_block(None, 256, 512, None, 512, None, 256, 0, None, 0, None) == 0
    assert L.wq_gemm_lut3(None, 48, 512, None, 512, None, 48, 0, None, 0, None) == 0
    assert L.wq_gemm_lut3_dense(None, 48, 512, None, 512, None, 48, 0, None, 0, None) == 0


@pytest.mark.parametrize("path,expect", [(3, 9), (-1, 9)])
def test_bad_path(path, expect):
    assert L.wq_gemm_fp8_block_path(P, 256, 512, P, 512, P, 256, 1, P, BIG, path, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, 48, 512, P, 512, P, 48, 1, P, BIG), 1),
    ((P, 40, 512, P, 512, P, 48, 1, P, BIG), 2),
    ((P, 48, 512, P, 512, P, 47, 1, P, BIG), 3),
    ((P, 48, 512, P, 500, P, 48, 1, P, BIG), 3),
])
def test_lut_gemm_validation(args, expect):
    assert L.wq_gemm_lut3(*args, None) == expect
    assert L.wq_gemm_lut3_dense(*args, None) == expect


def test_lut_has_no_gemv_path():
    # the GEMV arm is FP8-only; asking for it on LUT weights is refused by the
    # Python binding's path argument only for FP8, so check the C path code
    assert L.wq_gemm_fp8_block_path(P, 256, 512, P, 512, P, 256, 5, P, BIG, 1, None) == 9   # GEMV beyond M=4


@pytest.mark.parametrize("call,expect", [
    (lambda: L.wq_pack_fp8_block(None, 512, P, 256, 512, P, None), 1),
    (lambda: L.wq_pack_fp8_block(P, 511, P, 256, 512, P, None), 3),
    (lambda: L.wq_pack_fp8_block(P, 512, P, 255, 512, P, None), 2),
    (lambda: L.wq_pack_fp8_block(P, 512, P, 256, 512, P + 4, None), 8),
    (lambda: L.wq_pack_lut3(P, 512, None, P, 48, 512, P, None), 1),
    (lambda: L.wq_pack_lut3(P, 100, P, P, 48, 512, P, None), 3),
    (lambda: L.wq_pack_lut3(P, 512, P, P, 50, 512, P, None), 2),
    (lambda: L.wq_unpack_fp8_block(None, 256, 512, P, None), 1),
    (lambda: L.wq_unpack_fp8_block(P, 256, 500, P, None), 2),
    (lambda: L.wq_unpack_fp8_block_f32(P, 256, 512, P + 4, None), 8),
    (lambda: L.wq_unpack_lut3(P, 8, 512, P, None), 2),
    (lambda: L.wq_pack_lut3_dense(P, 512, None, P, 48, 512, P, None), 1),
    (lambda: L.wq_pack_lut3_dense(P, 100, P, P, 48, 512, P, None), 3),
    (lambda: L.wq_pack_lut3_dense(P, 512, P, P, 50, 512, P, None), 2),
    (lambda: L.wq_pack_lut3_dense(P, 512, P, P, 48, 512, P + 8, None), 8),
    (lambda: L.wq_unpack_lut3_dense(P, 8, 512, P, None), 2),
    (lambda: L.wq_unpack_lut3_dense(None, 16, 512, P, None), 1),
])
def test_pack_unpack_validation(call, expect):
    assert call() == expect


def test_w8a8_sizes_and_validation():
    assert wq.wq_x_fp8_packed_bytes(1, 128) == 16 * 128 + 4 * 16
    assert wq.wq_x_fp8_packed_bytes(17, 5120) == 32 * 5120 + 4 * 32 * 40
    assert wq.wq_x_fp8_packed_bytes(16, 100) == 0
    assert wq.wq_x_fp8_packed_bytes(0, 128) == 0
    assert wq.wq_x_fp8_packed_bytes(1 << 20, 4096) == 0                       # 2 GiB or more
    # (x, ldx, M, K, xq)
    assert L.wq_quantize_x_fp8(None, 512, 0, 512, None, None) == 0             # M == 0: no-op
    assert L.wq_quantize_x_fp8(None, 512, 4, 512, P, None) == 1
    assert L.wq_quantize_x_fp8(P, 511, 4, 512, P, None) == 3
    assert L.wq_quantize_x_fp8(P, 512, 4, 500, P, None) == 2
    assert L.wq_quantize_x_fp8(P, 516, 4, 512, P, None) == 8
    assert L.wq_quantize_x_fp8(P + 2, 512, 4, 512, P, None) == 8
    # (packed, N, K, xq, M, y, ldy, ws, ws_bytes)
    assert L.wq_gemm_fp8_w8a8(None, 256, 512, None, 0, None, 256, None, 0, None) == 0
    assert L.wq_gemm_fp8_w8a8(None, 256, 512, P, 4, P, 256, None, 0, None) == 1
    assert L.wq_gemm_fp8_w8a8(P, 200, 512, P, 4, P, 256, None, 0, None) == 2    # N % 128
    assert L.wq_gemm_fp8_w8a8(P, 256, 500, P, 4, P, 256, None, 0, None) == 2
    assert L.wq_gemm_fp8_w8a8(P, 256, 512, P, -1, P, 256, None, 0, None) == 2
    assert L.wq_gemm_fp8_w8a8(P, 256, 512, P, 4, P, 255, None, 0, None) == 3
    assert L.wq_gemm_fp8_w8a8(P, 256, 512, P + 8, 4, P, 256, None, 0, None) == 8
    assert L.wq_gemm_fp8_w8a8(P, 256, 512, P, 4, P + 1, 256, None, 0, None) == 8
    assert L.wq_unpack_x_fp8(P, 4, 512, P, P + 2, None) == 8
    assert L.wq_unpack_x_fp8(None, 4, 512, P, P, None) == 1


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
def test_valid_call_without_device_reports_hip_error():
    # arguments pass every host check; with no GPU the device query fails cleanly
    assert L.wq_gemm_fp8_block(P, 256, 512, P, 512, P, 256, 1, P, BIG, None) == 7
    assert L.wq_gemm_lut3(P, 48, 512, P, 512, P, 48, 4, P, BIG, None) == 7
    assert L.wq_gemm_lut3_dense(P, 48, 512, P, 512, P, 48, 4, P, BIG, None) == 7
    assert L.wq_gemm_fp8_w8a8(P, 256, 512, P, 4, P, 256, None, 0, None) == 7
    assert L.wq_quantize_x_fp8(P, 512, 4, 512, P, None) == 7
    assert L.wq_pack_fp8_block(P, 512, P, 256, 512, P, None) == 7


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
def test_large_stride_within_limits_passes_validation():
    # 31 rows of 2^26 BF16 elements + 1 KiB: just under 4 GiB; one row of any
    # stride.  The calls get past validation and fail only for want of a device
    assert L.wq_gemm_fp8_block(P, 256, 512, P, 1 << 26, P, 256, 32, P, BIG, None) == 7
    assert L.wq_gemm_fp8_block(P, 256, 512, P, 1 << 30, P, 256, 1, P, BIG, None) == 7


def test_noalloc_validates_before_the_device():
    """The no-allocation GEMM: M == 0 queues nothing; host validation errors come
    before any device work; the scratch bound is a constant."""
    assert wq.wq_noalloc_scratch_bytes() == 4 << 20
    f = wq.lib.wq_gemm_fp8_block_noalloc
    assert f(None, 256, 512, None, 512, None, 256, 0, None) == 0                    # M == 0
    assert f(None, 256, 512, None, 512, None, 256, 1, None) == 1                    # WQ_ERR_NULL
    assert f(16, 256, 500, 16, 512, 16, 256, 1, None) == 2                          # K % 128
    assert f(16, 256, 512, 16, 256, 16, 256, 1, None) == 3                          # ldx < K
    assert f(16, 256, 512, 16, 512, 16, 256, 33, None) == 2                         # M > 32
    assert wq.wq_status_str(wq.WQ_ERR_SCRATCH).startswith("WQ_ERR_SCRATCH")
