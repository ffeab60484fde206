"""libwq: decode-phase weight-only-quantized GEMM for MI355X (gfx950).

The compute path is the HIP library ``libwq.so`` built from ``csrc/``; this
package is only its Python binding (argument marshalling through ctypes, with
torch tensors supplying device memory and streams).  There is no fallback: if
the library is missing, importing :mod:`weight_only_quantized_fp8_amd.wq`
raises.
"""
from .wq import *  # noqa: F401,F403
from .wq import __all__  # noqa: F401
