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


def test_c_program_acceptance_rule_selftest():
    """The C program's own floor and element rule hold at the pinned points."""
    if not os.path.exists(BIN):
        pytest.skip("tests/c_abi/wq_c_smoke not built (__graft_entry__.build())")
    r = subprocess.run([BIN, "--selftest"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK: 0 failed checks (self-test)" in r.stdout


C_MUTANTS = [
    ("floor_no_sqrt", "1e-3 * sqrt((double)K) * xmax * wmax", "1e-3 * (double)K * xmax * wmax"),
    ("floor_coef_x10", "1e-3 * sqrt((double)K) * xmax * wmax", "1e-2 * sqrt((double)K) * xmax * wmax"),
    ("floor_drops_w", "1e-3 * sqrt((double)K) * xmax * wmax", "1e-3 * sqrt((double)K) * xmax"),
    ("rule_and", "isfinite(g) && (ulp_ok || abs_ok)", "isfinite(g) && (ulp_ok && abs_ok)"),
    ("ulp_3", "bf16_ord(wqo_bf16_rne(r))) <= 2", "bf16_ord(wqo_bf16_rne(r))) <= 3"),
    ("floor_strict", "fabs(g - r) <= floor_abs", "fabs(g - r) < floor_abs"),
    ("inf_allowed", "isfinite(g) && (ulp_ok || abs_ok)", "(ulp_ok || abs_ok)"),
    ("f16_raw", "is_f16 ? wqo_bf16_rne(g) : gb", "gb"),
]


@pytest.mark.parametrize("mid,find,repl", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_program_rule_mutant_is_caught(tmp_path, mid, find, repl):
    """A broken copy of the C program's acceptance rule fails its self-test."""
    libdir = os.path.join(ROOT, "weight_only_quantized_fp8_amd")
    if not os.path.exists(os.path.join(libdir, "libwq.so")) or not os.path.exists(
            os.path.join(ROOT, "oracle", "liboracle.so")):
        pytest.skip("libraries not built")
    with open(os.path.join(CDIR, "wq_c_smoke.c")) as f:
        text = f.read()
    assert text.count(find) == 1, "mutation anchor not found once: %r" % find
    src = tmp_path / ("%s.c" % mid)
    src.write_text(text.replace(find, repl))
    out = tmp_path / mid
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                           str(src), "-o", str(out), "-L", libdir, "-lwq",
                           "-L", os.path.join(ROOT, "oracle"), "-loracle",
                           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
                           "-Wl,-rpath,%s:%s:%s" % (libdir, os.path.join(ROOT, "oracle"), os.path.join(rocm, "lib"))])
    r = subprocess.run([str(out), "--selftest"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1, "mutant %s passed the self-test: %s" % (mid, r.stdout + r.stderr)
