"""The C-only smoke program of the boundary on the device: FP8 GEMMs on both
paths (M = 1, 4, 5, 16, 32) and LUT GEMMs in both layouts (M = 1, 7, 16, 20),
every output checked against the oracle, plus validation errors and the LUT
packer's code check -- all through include/wq.h from C, no Python on the
call path.  The program is built on the CPU by __graft_entry__.build()."""
import os
import subprocess

import pytest

import gpu_util as U

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "wq_c_smoke")


def test_c_program_passes_on_the_device():
    if not os.path.exists(BIN):
        pytest.skip("tests/c_abi/wq_c_smoke is not built (__graft_entry__.build() builds it; "
                    "tests/test_c_abi.py checks that it compiles)")
    U.note("c abi smoke program")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK: 0 failed checks" in r.stdout
