"""ctypes binding of include/wq.h.

Every ``wq_*`` function here has the name, argument order and meaning of the C
function it wraps; tensors stand in for device pointers and their leading
dimensions, and a non-OK status raises :class:`WqError`.  A few helpers
(``alloc_*``, ``workspace``, ``pack_*``/``gemm_*``) allocate outputs with torch.
Nothing here computes: every step runs in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "WqError", "LIB_PATH", "lib",
    "WQ_OK", "WQ_FMT_FP8_BLOCK", "WQ_FMT_LUT3", "WQ_PATH_AUTO", "WQ_PATH_GEMV", "WQ_PATH_MFMA",
    "wq_status_str", "wq_packed_format_version", "wq_set_tuning", "wq_set_kparts", "wq_set_w8a8_stages",
    "wq_fp8_block_packed_bytes", "wq_pack_fp8_block", "wq_gemm_fp8_block", "wq_gemm_fp8_block_path",
    "wq_gemm_fp8_block_noalloc", "wq_noalloc_scratch_bytes", "WQ_ERR_SCRATCH",
    "wq_lut3_packed_bytes", "wq_pack_lut3", "wq_gemm_lut3",
    "WQ_FMT_LUT3_DENSE", "wq_lut3_dense_packed_bytes", "wq_pack_lut3_dense", "wq_gemm_lut3_dense",
    "wq_unpack_lut3_dense", "pack_lut3_dense", "gemm_lut3_dense",
    "wq_x_fp8_packed_bytes", "wq_w8a8_workspace_bytes", "wq_quantize_x_fp8", "wq_gemm_fp8_w8a8", "wq_unpack_x_fp8", "quantize_x_fp8",
    "gemm_fp8_w8a8",
    "wq_gemm_workspace_bytes", "wq_unpack_fp8_block", "wq_unpack_fp8_block_f32", "wq_unpack_lut3",
    "wq_query_gemm_plan", "wq_query_w8a8_plan",
    "workspace", "pack_fp8", "pack_lut3", "gemm_fp8", "gemm_lut3",
]

# torch ships its own HIP runtime under the same soname as the system one
# (libamdhip64.so.7).  Loading torch first makes libwq bind to that already
# loaded runtime, so torch's device pointers and streams are valid in libwq's
# calls; loading libwq first would bring in a second, separate runtime.
import torch  # noqa: E402,F401  (must precede the CDLL below)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libwq.so is not built (%s); run __graft_entry__.build() or "
                      "python weight_only_quantized_fp8_amd/build.py" % LIB_PATH)
lib = ctypes.CDLL(LIB_PATH)

WQ_OK = 0
WQ_ERR_SCRATCH = 10
WQ_FMT_FP8_BLOCK, WQ_FMT_LUT3, WQ_FMT_LUT3_DENSE = 0, 1, 2
WQ_PATH_AUTO, WQ_PATH_GEMV, WQ_PATH_MFMA = 0, 1, 2

_P, _I64, _SZ, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
_SIGS = {
    "wq_status_str": (ctypes.c_char_p, [_INT]),
    "wq_packed_format_version": (_INT, []),
    "wq_set_tuning": (_INT, [_INT, _INT, _INT, _INT]),
    "wq_set_kparts": (_INT, [_INT]),
    "wq_set_w8a8_stages": (_INT, [_INT]),
    "wq_fp8_block_packed_bytes": (_SZ, [_I64, _I64]),
    "wq_pack_fp8_block": (_INT, [_P, _I64, _P, _I64, _I64, _P, _P]),
    "wq_gemm_fp8_block": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _P, _SZ, _P]),
    "wq_gemm_fp8_block_path": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _P, _SZ, _INT, _P]),
    "wq_gemm_fp8_block_noalloc": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _P]),
    "wq_noalloc_scratch_bytes": (_SZ, []),
    "wq_lut3_packed_bytes": (_SZ, [_I64, _I64]),
    "wq_pack_lut3": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "wq_gemm_lut3": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _P, _SZ, _P]),
    "wq_lut3_dense_packed_bytes": (_SZ, [_I64, _I64]),
    "wq_pack_lut3_dense": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "wq_gemm_lut3_dense": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _P, _SZ, _P]),
    "wq_unpack_lut3_dense": (_INT, [_P, _I64, _I64, _P, _P]),
    "wq_x_fp8_packed_bytes": (_SZ, [_I64, _I64]),
    "wq_w8a8_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "wq_quantize_x_fp8": (_INT, [_P, _I64, _I64, _I64, _P, _P]),
    "wq_gemm_fp8_w8a8": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _SZ, _P]),
    "wq_unpack_x_fp8": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "wq_gemm_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64]),
    "wq_unpack_fp8_block": (_INT, [_P, _I64, _I64, _P, _P]),
    "wq_unpack_fp8_block_f32": (_INT, [_P, _I64, _I64, _P, _P]),
    "wq_unpack_lut3": (_INT, [_P, _I64, _I64, _P, _P]),
    "wq_query_gemm_plan": (_INT, [_INT, _INT, _I64, _I64, _I64, _INT, _INT, ctypes.POINTER(_INT)]),
    "wq_query_w8a8_plan": (_INT, [_I64, _I64, _I64, _INT, _INT, ctypes.POINTER(_INT)]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class WqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, wq_status_str(status)))


def _check(st: int, where: str) -> None:
    if st != WQ_OK:
        raise WqError(st, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr() or None


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


# ------------------------------------------------------------- raw C calls

def wq_status_str(status: int) -> str:
    return lib.wq_status_str(int(status)).decode()


def wq_packed_format_version() -> int:
    return lib.wq_packed_format_version()


def wq_set_tuning(nt: int = 0, sn: int = 0, split: int = 0, waves_per_cu: int = 0) -> None:
    _check(lib.wq_set_tuning(nt, sn, split, waves_per_cu), "wq_set_tuning")


def wq_set_kparts(kp: int = 0) -> None:
    _check(lib.wq_set_kparts(kp), "wq_set_kparts")


def wq_set_w8a8_stages(stages: int = 0) -> None:
    _check(lib.wq_set_w8a8_stages(stages), "wq_set_w8a8_stages")


def wq_fp8_block_packed_bytes(N: int, K: int) -> int:
    return lib.wq_fp8_block_packed_bytes(N, K)


def wq_lut3_packed_bytes(N: int, K: int) -> int:
    return lib.wq_lut3_packed_bytes(N, K)


def wq_lut3_dense_packed_bytes(N: int, K: int) -> int:
    return lib.wq_lut3_dense_packed_bytes(N, K)


def wq_gemm_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return lib.wq_gemm_workspace_bytes(fmt, M, N, K)


def wq_pack_fp8_block(w_e4m3, scales, N: int, K: int, packed, stream=None) -> None:
    _check(lib.wq_pack_fp8_block(_ptr(w_e4m3), _ld(w_e4m3), _ptr(scales), N, K, _ptr(packed), _stream(stream)),
           "wq_pack_fp8_block")


def wq_gemm_fp8_block(packed, N: int, K: int, x, y, M: int, workspace=None, stream=None) -> None:
    _check(lib.wq_gemm_fp8_block(_ptr(packed), N, K, _ptr(x), _ld(x), _ptr(y), _ld(y), M, _ptr(workspace),
                                 _nbytes(workspace), _stream(stream)),
           "wq_gemm_fp8_block")


def wq_gemm_fp8_block_path(packed, N: int, K: int, x, y, M: int, workspace=None, path: int = WQ_PATH_AUTO,
                           stream=None) -> None:
    _check(lib.wq_gemm_fp8_block_path(_ptr(packed), N, K, _ptr(x), _ld(x), _ptr(y), _ld(y), M, _ptr(workspace),
                                      _nbytes(workspace), path, _stream(stream)),
           "wq_gemm_fp8_block_path")


def wq_gemm_fp8_block_noalloc(packed, N: int, K: int, x, y, M: int, stream=None) -> None:
    _check(lib.wq_gemm_fp8_block_noalloc(_ptr(packed), N, K, _ptr(x), _ld(x), _ptr(y), _ld(y), M,
                                         _stream(stream)), "wq_gemm_fp8_block_noalloc")


def wq_noalloc_scratch_bytes() -> int:
    return lib.wq_noalloc_scratch_bytes()


def wq_pack_lut3(codes, qmap, scales, N: int, K: int, packed, stream=None) -> None:
    _check(lib.wq_pack_lut3(_ptr(codes), _ld(codes), _ptr(qmap), _ptr(scales), N, K, _ptr(packed),
                            _stream(stream)), "wq_pack_lut3")


def wq_gemm_lut3(packed, N: int, K: int, x, y, M: int, workspace=None, stream=None) -> None:
    _check(lib.wq_gemm_lut3(_ptr(packed), N, K, _ptr(x), _ld(x), _ptr(y), _ld(y), M, _ptr(workspace),
                            _nbytes(workspace), _stream(stream)), "wq_gemm_lut3")


def wq_pack_lut3_dense(codes, qmap, scales, N: int, K: int, packed, stream=None) -> None:
    _check(lib.wq_pack_lut3_dense(_ptr(codes), _ld(codes), _ptr(qmap), _ptr(scales), N, K, _ptr(packed),
                                  _stream(stream)), "wq_pack_lut3_dense")


def wq_gemm_lut3_dense(packed, N: int, K: int, x, y, M: int, workspace=None, stream=None) -> None:
    _check(lib.wq_gemm_lut3_dense(_ptr(packed), N, K, _ptr(x), _ld(x), _ptr(y), _ld(y), M, _ptr(workspace),
                                  _nbytes(workspace), _stream(stream)), "wq_gemm_lut3_dense")


def wq_unpack_fp8_block(packed, N: int, K: int, w_bf16, stream=None) -> None:
    _check(lib.wq_unpack_fp8_block(_ptr(packed), N, K, _ptr(w_bf16), _stream(stream)), "wq_unpack_fp8_block")


def wq_unpack_fp8_block_f32(packed, N: int, K: int, w_f32, stream=None) -> None:
    _check(lib.wq_unpack_fp8_block_f32(_ptr(packed), N, K, _ptr(w_f32), _stream(stream)),
           "wq_unpack_fp8_block_f32")


def wq_unpack_lut3(packed, N: int, K: int, w_f16, stream=None) -> None:
    _check(lib.wq_unpack_lut3(_ptr(packed), N, K, _ptr(w_f16), _stream(stream)), "wq_unpack_lut3")


def wq_unpack_lut3_dense(packed, N: int, K: int, w_f16, stream=None) -> None:
    _check(lib.wq_unpack_lut3_dense(_ptr(packed), N, K, _ptr(w_f16), _stream(stream)), "wq_unpack_lut3_dense")


def wq_x_fp8_packed_bytes(M: int, K: int) -> int:
    return lib.wq_x_fp8_packed_bytes(M, K)


def wq_w8a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib.wq_w8a8_workspace_bytes(M, N, K)


def wq_quantize_x_fp8(x, M: int, K: int, xq, stream=None) -> None:
    _check(lib.wq_quantize_x_fp8(_ptr(x), _ld(x), M, K, _ptr(xq), _stream(stream)), "wq_quantize_x_fp8")


def wq_gemm_fp8_w8a8(packed, N: int, K: int, xq, M: int, y, workspace=None, stream=None) -> None:
    _check(lib.wq_gemm_fp8_w8a8(_ptr(packed), N, K, _ptr(xq), M, _ptr(y), _ld(y), _ptr(workspace),
                                _nbytes(workspace), _stream(stream)), "wq_gemm_fp8_w8a8")


def wq_query_gemm_plan(fmt: int, M: int, N: int, K: int, cu: int, with_workspace: bool = False,
                       path: int = WQ_PATH_AUTO) -> dict:
    """Host-only: the plan a decode GEMM call would take on a device with `cu`
    compute units (no device is touched)."""
    out = (_INT * 6)()
    _check(lib.wq_query_gemm_plan(fmt, path, M, N, K, cu, int(bool(with_workspace)), out), "wq_query_gemm_plan")
    return dict(path=out[0], nt=out[1], sn=out[2], split=out[3], kparts=out[4], launches=out[5])


def wq_query_w8a8_plan(M: int, N: int, K: int, cu: int, with_workspace: bool = False) -> dict:
    """Host-only: the tile and K parts a W8A8 call would take on a device with
    `cu` compute units (no device is touched).  `band` is the number of leading
    columns on that plan (N when the call is one launch); the remaining columns
    run as a second launch on `tail` = (tile rows, tile columns, K parts), else
    None."""
    out = (_INT * 8)()
    _check(lib.wq_query_w8a8_plan(M, N, K, cu, int(bool(with_workspace)), out), "wq_query_w8a8_plan")
    tail = (out[5], out[6], out[7]) if out[4] < N else None
    return dict(tile=(out[0], out[1]), kparts=out[2], streaming=bool(out[3]), band=out[4], tail=tail)


def wq_unpack_x_fp8(xq, M: int, K: int, codes, scales, stream=None) -> None:
    _check(lib.wq_unpack_x_fp8(_ptr(xq), M, K, _ptr(codes), _ptr(scales), _stream(stream)), "wq_unpack_x_fp8")


# -------------------------------------------------------- torch helpers

def workspace(fmt: int, N: int, K: int, device="cuda"):
    """Workspace for GEMMs of this format and shape (any M, any path); empty (passed
    as NULL) when the shape keeps K inside one work-group."""
    import torch
    nbytes = wq_gemm_workspace_bytes(fmt, 1, N, K)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def pack_fp8(codes, scales, stream=None):
    """Pack E4M3 codes [N, K] (uint8, cuda) and FP32 block scales into a new buffer."""
    import torch
    N, K = codes.shape[0], codes.shape[1]
    packed = torch.empty(wq_fp8_block_packed_bytes(N, K), dtype=torch.uint8, device=codes.device)
    wq_pack_fp8_block(codes, scales, N, K, packed, stream)
    return packed


def pack_lut3(codes, qmap, scales, stream=None):
    """Pack 3-bit codes [N, K] (uint8), FP16 map [8] and FP16 group scales into a new buffer."""
    import torch
    N, K = codes.shape[0], codes.shape[1]
    packed = torch.empty(wq_lut3_packed_bytes(N, K), dtype=torch.uint8, device=codes.device)
    wq_pack_lut3(codes, qmap, scales, N, K, packed, stream)
    return packed


def gemm_fp8(packed, N: int, K: int, x, ws=None, path: int = WQ_PATH_AUTO, stream=None):
    """y [M, N] (bfloat16) = x [M, K] (bfloat16) . dequant(W)^T."""
    import torch
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    wq_gemm_fp8_block_path(packed, N, K, x, y, M, ws, path, stream)
    return y


def gemm_lut3(packed, N: int, K: int, x, ws=None, stream=None):
    """y [M, N] (float16) = x [M, K] (float16) . dequant(W)^T."""
    import torch
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    wq_gemm_lut3(packed, N, K, x, y, M, ws, stream)
    return y


def pack_lut3_dense(codes, qmap, scales, stream=None):
    """Pack 3-bit codes [N, K] (uint8), FP16 map [8] and FP16 group scales densely (3 bits a code)."""
    import torch
    N, K = codes.shape[0], codes.shape[1]
    packed = torch.empty(wq_lut3_dense_packed_bytes(N, K), dtype=torch.uint8, device=codes.device)
    wq_pack_lut3_dense(codes, qmap, scales, N, K, packed, stream)
    return packed


def gemm_lut3_dense(packed, N: int, K: int, x, ws=None, stream=None):
    """y [M, N] (float16) = x [M, K] (float16) . dequant(W)^T for a densely packed matrix."""
    import torch
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    wq_gemm_lut3_dense(packed, N, K, x, y, M, ws, stream)
    return y


def quantize_x_fp8(x, stream=None):
    """Packed FP8 activations (uint8 buffer) of BF16 x [M, K]."""
    import torch
    M, K = x.shape[0], x.shape[1]
    xq = torch.empty(wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=x.device)
    wq_quantize_x_fp8(x, M, K, xq, stream)
    return xq


def gemm_fp8_w8a8(packed, N: int, K: int, xq, M: int, ws=None, stream=None):
    """y [M, N] (bfloat16) = dequant(xq) . dequant(W)^T (ws: optional workspace of
    wq_w8a8_workspace_bytes(M, N, K) bytes)."""
    import torch
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    wq_gemm_fp8_w8a8(packed, N, K, xq, M, y, ws, stream)
    return y
