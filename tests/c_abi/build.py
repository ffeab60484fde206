"""Build the C-only smoke program of the libwq boundary (test infrastructure).

gcc, C11, against include/wq.h and the HIP runtime's C API; links libwq.so
and the oracle's liboracle.so through run paths relative to the binary, so
the program runs from any checkout without an environment.  Needs both
libraries built first.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "wq_c_smoke.c")
BIN = os.path.join(HERE, "wq_c_smoke")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "weight_only_quantized_fp8_amd"), "-lwq",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../weight_only_quantized_fp8_amd:$ORIGIN/../../oracle:" + os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
    sys.exit(0)
