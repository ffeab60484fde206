"""CPU oracle for the decode-phase weight-only-quantized GEMM (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library never does, and this package
never imports the library: they share no code.

The arithmetic lives in ``oracle.c`` (plain C, binary64, one accumulator per
output walking k in increasing order); this module only marshals numpy arrays
through ctypes.  ``compare.py`` holds the acceptance rule.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC", "-pthread"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


class using:
    """Context manager that points this module at another build of oracle.c.

    Used only by the mutation tests, which compile deliberately broken copies of
    the oracle and check that the pins catch them."""

    def __init__(self, path: str):
        self.path = path
        self.prev = None

    def __enter__(self):
        global _lib
        _load()
        self.prev = _lib
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = _bind(_LIB_PATH)
    return _lib


def _declare(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.wqo_e4m3_value.restype = ctypes.c_double
    lib.wqo_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.wqo_f16_value.restype = ctypes.c_double
    lib.wqo_f16_value.argtypes = [ctypes.c_uint16]
    lib.wqo_bf16_value.restype = ctypes.c_double
    lib.wqo_bf16_value.argtypes = [ctypes.c_uint16]
    lib.wqo_f16_rne.restype = ctypes.c_uint16
    lib.wqo_f16_rne.argtypes = [ctypes.c_double]
    lib.wqo_bf16_rne.restype = ctypes.c_uint16
    lib.wqo_bf16_rne.argtypes = [ctypes.c_double]
    for name in ("wqo_f16_rne_array", "wqo_bf16_rne_array", "wqo_e4m3_value_array",
                 "wqo_f16_value_array", "wqo_bf16_value_array"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [P, I64, P]
    lib.wqo_dequant_fp8.restype = ctypes.c_int
    lib.wqo_dequant_fp8.argtypes = [P, I64, P, I64, I64, P]
    lib.wqo_dequant_lut3.restype = ctypes.c_int
    lib.wqo_dequant_lut3.argtypes = [P, I64, P, P, I64, I64, P]
    lib.wqo_gemm_fp8.restype = ctypes.c_int
    lib.wqo_gemm_fp8.argtypes = [P, I64, P, I64, P, I64, I64, I64, P, I64, P, ctypes.c_int]
    lib.wqo_gemm_lut3.restype = ctypes.c_int
    lib.wqo_gemm_lut3.argtypes = [P, I64, P, I64, P, P, I64, I64, I64, P, I64, P, ctypes.c_int]
    lib.wqo_e4m3_rne.restype = ctypes.c_uint8
    lib.wqo_e4m3_rne.argtypes = [ctypes.c_float]
    lib.wqo_quantize_x_fp8.restype = ctypes.c_int
    lib.wqo_quantize_x_fp8.argtypes = [P, I64, I64, I64, P, P]
    lib.wqo_gemm_w8a8.restype = ctypes.c_int
    lib.wqo_gemm_w8a8.argtypes = [P, I64, P, P, I64, P, I64, I64, I64, P, I64, P, ctypes.c_int]


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


# ------------------------------------------------------------------ scalars

def e4m3_value(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().wqo_e4m3_value_array(_ptr(c), c.size, _ptr(out))
    return out


def f16_value(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().wqo_f16_value_array(_ptr(b), b.size, _ptr(out))
    return out


def bf16_value(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().wqo_bf16_value_array(_ptr(b), b.size, _ptr(out))
    return out


def f16_rne(v) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().wqo_f16_rne_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_rne(v) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().wqo_bf16_rne_array(_ptr(a), a.size, _ptr(out))
    return out


# ------------------------------------------------------------------ weights

def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w[n,k] = e4m3(q[n,k]) * s[n/128][k/128] as float64 [N, K]."""
    q = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    N, K = q.shape
    out = np.empty((N, K), dtype=np.float64)
    rc = _load().wqo_dequant_fp8(_ptr(q), K, _ptr(s), N, K, _ptr(out))
    if rc:
        raise ValueError("wqo_dequant_fp8 failed: %d" % rc)
    return out


def dequant_lut3(codes: np.ndarray, qmap: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w[n,k] = fp16_rne(qmap[c[n,k]] * g[n][k/128]) as float64 [N, K]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    qm = np.ascontiguousarray(qmap, dtype=np.uint16)
    g = np.ascontiguousarray(scales, dtype=np.uint16)
    N, K = c.shape
    out = np.empty((N, K), dtype=np.float64)
    rc = _load().wqo_dequant_lut3(_ptr(c), K, _ptr(qm), _ptr(g), N, K, _ptr(out))
    if rc:
        raise ValueError("wqo_dequant_lut3 failed: %d" % rc)
    return out


# --------------------------------------------------------------------- GEMM

def _cols_arg(cols):
    if cols is None:
        return None, None
    c = np.ascontiguousarray(cols, dtype=np.int64)
    return c, _ptr(c)


def gemm_fp8(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, K: int | None = None,
             cols=None, nthreads: int | None = None) -> np.ndarray:
    """y64 [M, N] (or [M, len(cols)]) for BF16 x bits [M, ldx] and FP8 codes [N, ldq]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    M, ldx = x.shape
    N, ldq = q.shape
    K = ldq if K is None else K
    c, cp = _cols_arg(cols)
    nc = N if c is None else c.size
    y = np.empty((M, nc), dtype=np.float64)
    rc = _load().wqo_gemm_fp8(_ptr(x), ldx, _ptr(q), ldq, _ptr(s), M, N, K, cp, nc, _ptr(y),
                              nthreads or default_threads())
    if rc:
        raise ValueError("wqo_gemm_fp8 failed: %d" % rc)
    return y


def gemm_lut3(x_bits: np.ndarray, codes: np.ndarray, qmap: np.ndarray, scales: np.ndarray,
              K: int | None = None, cols=None, nthreads: int | None = None) -> np.ndarray:
    """y64 [M, N] (or [M, len(cols)]) for FP16 x bits [M, ldx] and 3-bit codes [N, ldc]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    cc = np.ascontiguousarray(codes, dtype=np.uint8)
    qm = np.ascontiguousarray(qmap, dtype=np.uint16)
    g = np.ascontiguousarray(scales, dtype=np.uint16)
    M, ldx = x.shape
    N, ldc = cc.shape
    K = ldc if K is None else K
    c, cp = _cols_arg(cols)
    nc = N if c is None else c.size
    y = np.empty((M, nc), dtype=np.float64)
    rc = _load().wqo_gemm_lut3(_ptr(x), ldx, _ptr(cc), ldc, _ptr(qm), _ptr(g), M, N, K, cp, nc,
                               _ptr(y), nthreads or default_threads())
    if rc:
        raise ValueError("wqo_gemm_lut3 failed: %d" % rc)
    return y


# ------------------------------------------------------------------- W8A8

def e4m3_rne(v) -> np.ndarray:
    """Nearest E4M3FN code (ties to even) of each binary32 value, |v| <= 448."""
    a = np.ascontiguousarray(v, dtype=np.float32).ravel()
    lib = _load()
    return np.array([lib.wqo_e4m3_rne(float(t)) for t in a], dtype=np.uint8).reshape(np.shape(v))


def quantize_x_fp8(x_bits: np.ndarray, K: int | None = None):
    """(codes uint8 [M, K], scales float32 [M, K/128]) of BF16 x bits [M, ldx]:
    per (row, 128-K group) s = amax/448, codes = e4m3_rne(clamp(x/s, +-448))."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, ldx = x.shape
    K = ldx if K is None else K
    codes = np.empty((M, K), dtype=np.uint8)
    scales = np.empty((M, K // 128), dtype=np.float32)
    rc = _load().wqo_quantize_x_fp8(_ptr(x), ldx, M, K, _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("wqo_quantize_x_fp8 failed: %d" % rc)
    return codes, scales


def gemm_w8a8(x_codes: np.ndarray, x_scales: np.ndarray, codes: np.ndarray, scales: np.ndarray,
              K: int | None = None, cols=None, nthreads: int | None = None) -> np.ndarray:
    """y64 [M, N] (or [M, len(cols)]) for FP8 activations (codes [M, ldxq], scales
    [M, K/128]) and FP8 block-scaled weights (codes [N, ldq], scales [N/128, K/128])."""
    xq = np.ascontiguousarray(x_codes, dtype=np.uint8)
    sx = np.ascontiguousarray(x_scales, dtype=np.float32)
    q = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    M, ldxq = xq.shape
    N, ldq = q.shape
    K = ldq if K is None else K
    c, cp = _cols_arg(cols)
    nc = N if c is None else c.size
    y = np.empty((M, nc), dtype=np.float64)
    rc = _load().wqo_gemm_w8a8(_ptr(xq), ldxq, _ptr(sx), _ptr(q), ldq, _ptr(s), M, N, K, cp, nc, _ptr(y),
                               nthreads or default_threads())
    if rc:
        raise ValueError("wqo_gemm_w8a8 failed: %d" % rc)
    return y
