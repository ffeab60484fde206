"""Seeded synthetic inputs for the decode-phase weight-only-quantized GEMM.

This module only *draws* data and stores it in the formats the library consumes:
it encodes, it never decodes and it never multiplies weights by activations.
Both the CPU oracle and the GPU path read what it returns; neither shares any
other code with it.

Workload recipe (stands in for the trained checkpoints, activations and learned
maps the pages measure on, none of which are available):

* FP8 block-scaled weights -- the layer shapes of the dense-FFN and attention
  projections in the atlas ``m16_tc`` module docs (sections "WHY" and "WHY THE FFN
  ARM LOSES"): W ~ N(0, 0.02) drawn in float32, split into 128x128 blocks (the
  ``weight_block_size [128, 128]`` of the arc PR "FP8 bank conflict + the dispatch
  threshold's provenance"), per block scale s = amax/448 in float32, codes =
  E4M3FN round-to-nearest-even of clamp(W/s, -448, 448).  A block whose amax is
  0 gets s = 1 and all-zero codes.
* 3-bit LUT weights -- the 28672x8192 shape of the FLUTE ``optimized_w3`` PR
  ("Results"): codes uniform in 0..7 (one per byte, canonical row-major [N, K]),
  an 8-entry FP16 map = the sorted float16 roundings of 8 N(0,1) draws, FP16 group
  scales ~ U(0.005, 0.02) per (row, 128-wide K group).
* Activations x ~ N(0,1) in float32, rounded to BF16 (FP8 path) or FP16 (LUT path).

Random numbers come from ``numpy.random.Generator(PCG64(.))``: a matrix is drawn
in fixed chunks of 1024 rows, chunk i from ``SeedSequence(seed).spawn(...)[i]``,
so the values depend only on the seed and the shape (never on the thread count)
and large matrices can be drawn in parallel.  Stored dtypes are produced with
library conversions (torch's float8_e4m3fn / bfloat16 casts and numpy's float16
cast), all round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "SEEDS", "CONFIGS", "normal_matrix", "fp8_weights", "lut3_weights", "x_bf16", "x_f16",
    "bits_to_torch",
]

# Seeds per named workload; activations use seed + 100.
SEEDS = {
    "tiny": 1000, "gate_up": 1001, "down": 1002, "lut3": 1003,
    "attn_q": 1004, "attn_k": 1005, "attn_v": 1006, "attn_o": 1007,
    "lut3d": 1003,     # the "lut3" matrix and activations, stored densely (3 bits a code)
    "attn_qkv": 1008,  # the Q, K and V projections stacked into one 8192-row matrix
}

# name -> (format, N, K, M sweep); format "lut3d" is the LUT format with the
# codes stored at 3 bits each instead of one per nibble
CONFIGS = {
    "tiny":    ("fp8", 256, 512, (1,)),
    "gate_up": ("fp8", 17408, 5120, (1, 4, 8, 16)),
    "down":    ("fp8", 5120, 17408, (1, 8, 16, 32)),
    "lut3":    ("lut3", 28672, 8192, (1, 2, 4, 8, 16)),
    "attn_q":  ("fp8", 6144, 5120, (16,)),
    "attn_k":  ("fp8", 1024, 5120, (16,)),
    "attn_v":  ("fp8", 1024, 5120, (16,)),
    "attn_o":  ("fp8", 5120, 6144, (16,)),
    "lut3d":   ("lut3d", 28672, 8192, (1, 2, 4, 8, 16)),
    "attn_qkv": ("fp8", 8192, 5120, (16,)),
}

_BLOCK = 128
_E4M3_MAX = 448.0


_CHUNK_ROWS = 1024


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _chunked(seed: int, rows: int, fill) -> None:
    """Call fill(generator, r0, r1) for each 1024-row chunk, in parallel threads."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    n = (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    seqs = np.random.SeedSequence(seed).spawn(n)
    jobs = [(np.random.Generator(np.random.PCG64(seqs[i])), i * _CHUNK_ROWS, min(rows, (i + 1) * _CHUNK_ROWS))
            for i in range(n)]
    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: fill(*j), jobs))


def normal_matrix(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    """float32 [rows, cols] ~ N(0, std^2), chunk-seeded (see module doc)."""
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(g, r0, r1):
        g.standard_normal((r1 - r0, cols), dtype=np.float32, out=out[r0:r1])
        if std != 1.0:
            out[r0:r1] *= np.float32(std)
    _chunked(seed, rows, fill)
    return out


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """float32 array (already within +-448) -> E4M3FN code bytes, RNE (torch cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_weights(N: int, K: int, seed: int, std: float = 0.02, w: np.ndarray | None = None):
    """Return (codes uint8 [N, K], scales float32 [N/128, K/128]).

    ``w`` may supply the float32 matrix instead of the N(0, std) draw (used by
    tests that need structured values).
    """
    if N % _BLOCK or K % _BLOCK:
        raise ValueError("N and K must be multiples of 128 for 128x128 block scales")
    import torch
    if w is None:
        w = normal_matrix(N, K, seed, std)
    w = np.asarray(w, dtype=np.float32)
    nb, kb = N // _BLOCK, K // _BLOCK
    wt = torch.from_numpy(w)
    amax = wt.view(nb, _BLOCK, kb, _BLOCK).abs().amax(dim=(1, 3))                  # [nb, kb] float32
    scales = torch.where(amax > 0, amax / _E4M3_MAX, torch.ones_like(amax))        # float32 division
    q = (wt.view(nb, _BLOCK, kb, _BLOCK) / scales[:, None, :, None]).clamp_(-_E4M3_MAX, _E4M3_MAX)
    codes = q.reshape(N, K).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scales.numpy().astype(np.float32)


def lut3_weights(N: int, K: int, seed: int, g_lo: float = 0.005, g_hi: float = 0.02):
    """Return (codes uint8 [N, K] in 0..7, qmap uint16 FP16 bits [8], scales uint16 FP16 bits [N, K/128])."""
    if N % 16 or K % _BLOCK:
        raise ValueError("N must be a multiple of 16 and K of 128")
    r = _rng(seed)
    qmap = np.sort(r.standard_normal(8, dtype=np.float32).astype(np.float16))
    scales = r.uniform(g_lo, g_hi, size=(N, K // _BLOCK)).astype(np.float32).astype(np.float16)
    codes = np.empty((N, K), dtype=np.uint8)

    def fill(g, r0, r1):
        codes[r0:r1] = g.integers(0, 8, size=(r1 - r0, K), dtype=np.uint8)
    _chunked(seed + 7919, N, fill)
    return codes, qmap.view(np.uint16).copy(), scales.view(np.uint16).copy()


def x_bf16(M: int, K: int, seed: int, ld: int | None = None) -> np.ndarray:
    """BF16 bits uint16 [M, ld] (columns >= K are padding filled with a canary pattern)."""
    import torch
    ld = K if ld is None else ld
    x = normal_matrix(M, K, seed)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = np.full((M, ld), 0x7FC1, dtype=np.uint16)   # canary: a NaN payload
    out[:, :K] = bits
    return out


def x_f16(M: int, K: int, seed: int, ld: int | None = None) -> np.ndarray:
    """FP16 bits uint16 [M, ld] (padding columns hold a NaN canary)."""
    ld = K if ld is None else ld
    x = normal_matrix(M, K, seed).astype(np.float16)
    out = np.full((M, ld), 0x7E01, dtype=np.uint16)
    out[:, :K] = x.view(np.uint16)
    return out


def bits_to_torch(a: np.ndarray, device=None):
    """Wrap a numpy array (uint8/uint16/float32) as a torch tensor on ``device``."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy())
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t if device is None else t.to(device)
