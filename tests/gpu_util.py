"""Helpers shared by the GPU tests: run the HIP path through the C ABI on seeded
inputs and grade it against the CPU oracle.  Nothing here computes results:
the device side is libwq, the reference side is oracle/."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth
from oracle import compare

DEV = "cuda:0"


def wqmod():
    from weight_only_quantized_fp8_amd import wq
    return wq


def note(msg: str) -> None:
    """Print and flush what names the case before GPU work, so a failure that
    takes the process down still leaves the case on record."""
    print(msg, flush=True)
    sys.stdout.flush()


def t_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def t_u16(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV).view(dtype)


def t_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bits_of(t) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ FP8

def pack_fp8(codes, scales, ldw=None):
    wq = wqmod()
    N, K = codes.shape
    if ldw is not None and ldw > K:
        wide = np.zeros((N, ldw), dtype=np.uint8)
        wide[:, :K] = codes
        wide[:, K:] = 0x7F
        src = t_u8(wide)[:, :K]
    else:
        src = t_u8(codes)
    packed = torch.empty(wq.wq_fp8_block_packed_bytes(N, K), dtype=torch.uint8, device=DEV)
    wq.wq_pack_fp8_block(src, t_f32(scales), N, K, packed)
    return packed


def run_fp8(packed, N, K, xbits, M=None, path=0, ws=None, ldy=None, y_init=None):
    """xbits: uint16 [M, ldx] (ldx >= K).  ws: None (no workspace: every output
    reduced in its work-group), "auto" (wq.workspace for the shape: K parts
    where its plan splits K across work-groups) or a buffer.  Returns (y bits
    [M, N], full y buffer bits)."""
    wq = wqmod()
    M = xbits.shape[0] if M is None else M
    x = t_u16(xbits, torch.bfloat16)
    ldy = N if ldy is None else ldy
    y = torch.empty((max(M, 1), ldy), dtype=torch.bfloat16, device=DEV)
    if y_init is not None:
        y.copy_(t_u16(y_init, torch.bfloat16))
    ws = wq.workspace(wq.WQ_FMT_FP8_BLOCK, N, K, DEV) if isinstance(ws, str) else ws
    wq.wq_gemm_fp8_block_path(packed, N, K, x, y, M, ws, path)
    torch.cuda.synchronize()
    full = bits_of(y)
    return full[:M, :N], full


def floor_fp8(xbits, codes, scales, K):
    mx = float(np.abs(oracle.bf16_value(xbits[:, :K])).max())
    mw = 0.0
    for r0 in range(0, codes.shape[0], 2048):
        w = oracle.dequant_fp8(codes[r0:r0 + 2048], scales[r0 // 128:(r0 + 2048) // 128])
        mw = max(mw, float(np.nanmax(np.abs(w))))
    return compare.abs_floor(K, mx, mw)


def grade_fp8(ybits, xbits, codes, scales, K, cols=None, floor=None):
    y64 = oracle.gemm_fp8(xbits, codes, scales, K=K, cols=cols)
    if floor is None:
        floor = floor_fp8(xbits, codes, scales, K)
    yb = ybits if cols is None else ybits[:, cols]
    return compare.grade(yb, y64, floor, "bf16")


# ------------------------------------------------------------------ LUT3

def pack_lut3(codes, qmap, scales, dense=False):
    """dense: the 3-bit-per-code layout (wq_pack_lut3_dense) instead of nibbles."""
    wq = wqmod()
    N, K = codes.shape
    nbytes = (wq.wq_lut3_dense_packed_bytes if dense else wq.wq_lut3_packed_bytes)(N, K)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    (wq.wq_pack_lut3_dense if dense else wq.wq_pack_lut3)(
        t_u8(codes), t_u16(qmap, torch.float16), t_u16(scales, torch.float16), N, K, packed)
    return packed


def run_lut3(packed, N, K, xbits, M=None, ws=None, ldy=None, y_init=None, dense=False):
    """As run_fp8 for the LUT formats (dense: the 3-bit code layout)."""
    wq = wqmod()
    M = xbits.shape[0] if M is None else M
    x = t_u16(xbits, torch.float16)
    ldy = N if ldy is None else ldy
    y = torch.empty((max(M, 1), ldy), dtype=torch.float16, device=DEV)
    if y_init is not None:
        y.copy_(t_u16(y_init, torch.float16))
    fmt = wq.WQ_FMT_LUT3_DENSE if dense else wq.WQ_FMT_LUT3
    ws = wq.workspace(fmt, N, K, DEV) if isinstance(ws, str) else ws
    (wq.wq_gemm_lut3_dense if dense else wq.wq_gemm_lut3)(packed, N, K, x, y, M, ws)
    torch.cuda.synchronize()
    full = bits_of(y)
    return full[:M, :N], full


def floor_lut3(xbits, codes, qmap, scales, K):
    mx = float(np.abs(oracle.f16_value(xbits[:, :K])).max())
    mw = 0.0
    for r0 in range(0, codes.shape[0], 2048):
        w = oracle.dequant_lut3(codes[r0:r0 + 2048], qmap, scales[r0:r0 + 2048])
        mw = max(mw, float(np.abs(w).max()))
    return compare.abs_floor(K, mx, mw)


def grade_lut3(ybits, xbits, codes, qmap, scales, K, cols=None, floor=None):
    y64 = oracle.gemm_lut3(xbits, codes, qmap, scales, K=K, cols=cols)
    if floor is None:
        floor = floor_lut3(xbits, codes, qmap, scales, K)
    yb = ybits if cols is None else ybits[:, cols]
    return compare.grade(yb, y64, floor, "f16")


# Beyond the contract: at most this fraction of the outputs may lie beyond 2
# BF16 ULP (such outputs pass only through the absolute floor).  The floor is
# wide at large K (2.7% of the output RMS at the FFN gate/up size), so without
# this bound a fault that shifts outputs by a few per cent -- a wrong block
# scale, a lost K block -- could still pass element by element.  The atlas
# m16_tc docs' own M=32 receipt had 5 of 557,056 outputs over the budget, all
# cancellations.
# FP16 outputs below FP16's smallest normal are not counted: FP16's spacing
# there is coarser than 2 BF16 ULP, so even a correctly rounded value can be
# over the budget (Receipt.n_over_budget_resolvable).
OVER_BUDGET_FRAC = 1e-4
# rel_rms bounds by output type: BF16 rounding alone gives ~1.5e-3, FP16 ~2e-4
REL_RMS_MAX = {"bf16": 4e-3, "f16": 1e-3}


def check(r, what: str = "", out_dtype: str = "bf16", max_over: int | None = None) -> None:
    """Assert a receipt: every output within the contract, at most
    OVER_BUDGET_FRAC of them (or max_over) beyond 2 ULP, no sign flips,
    rel_rms bounded."""
    tag = ("%s: " % what if what else "") + str(r)
    assert r.ok, tag
    if max_over is None:
        max_over = int(OVER_BUDGET_FRAC * r.n)
    assert r.n_over_budget_resolvable <= max_over, "over budget: " + tag
    assert r.sign_flips == 0, tag
    assert np.isfinite(r.rel_rms) and r.rel_rms < REL_RMS_MAX[out_dtype], "rel_rms: " + tag


def sample_cols(N: int, seed: int, n: int = 768) -> np.ndarray:
    """Every column of the first and last 128, plus n random ones in between."""
    rng = np.random.Generator(np.random.PCG64(seed))
    mid = rng.choice(np.arange(128, max(128, N - 128)), size=min(n, max(0, N - 256)), replace=False)
    return np.unique(np.concatenate([np.arange(min(128, N)), np.arange(max(0, N - 128), N), mid]))


@functools.lru_cache(maxsize=4)
def config_inputs(name: str):
    fmt, N, K, Ms = synth.CONFIGS[name]
    seed = synth.SEEDS[name]
    if fmt == "fp8":
        codes, scales = synth.fp8_weights(N, K, seed)
        return fmt, N, K, Ms, (codes, scales)
    codes, qmap, g = synth.lut3_weights(N, K, seed)
    return fmt, N, K, Ms, (codes, qmap, g)
