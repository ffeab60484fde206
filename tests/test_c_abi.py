"""The boundary used from plain C: tests/c_abi/wq_c_smoke.c includes
include/wq.h as C11 (no C++ in the header), allocates device memory with the
HIP runtime's C API, packs and multiplies through the C ABI and checks every
output against the CPU oracle.  Here (CPU): it builds warning-free with
-Werror and, with no device, reports that and exits 2 without a GEMM call.
The GPU test runs it on the device."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CDIR = os.path.join(HERE, "c_abi")
BIN = os.path.join(CDIR, "wq_c_smoke")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_c_program_builds_as_c11_without_warnings(tmp_path):
    if not os.path.exists(os.path.join(ROOT, "weight_only_quantized_fp8_amd", "libwq.so")):
        pytest.skip("libwq.so not built")
    out = tmp_path / "wq_c_smoke"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                           os.path.join(CDIR, "wq_c_smoke.c"), "-o", str(out),
                           "-L", os.path.join(ROOT, "weight_only_quantized_fp8_amd"), "-lwq",
                           "-L", os.path.join(ROOT, "oracle"), "-loracle",
                           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm"])


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device exit")
def test_c_program_without_a_device_exits_2():
    if not os.path.exists(BIN):
        pytest.skip("tests/c_abi/wq_c_smoke not built (__graft_entry__.build())")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2, r.stdout + r.stderr
    assert "no HIP device" in r.stderr
