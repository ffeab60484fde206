"""Per-shape tiling sweep for libwq, gated on exactness.

    python -m weight_only_quantized_fp8_amd.tune --fmt fp8 --N 17408 --K 5120 --M 16

For one format and shape it runs every candidate tiling (tiles per wave,
column-waves sharing activations, waves per work-group) through the library's
own tuning hook (``wq_set_tuning``); with ``--kparts`` it also sweeps the
number of K parts split across work-groups (``wq_set_kparts``), passing each
call a workspace of ``wq_gemm_workspace_bytes``.  A candidate is timed only if its output
passes the library's tolerance against an FP32 reference built from the
library's own dequantised weights (``wq_unpack_*``) and a torch matmul: every
output within 2 BF16 ULP of the reference or within 1e-3*sqrt(K)*max|x|*max|w|.
The fastest passing candidates are printed, the best one in the form of a
per-shape table row (the per-shape dispatch of the FLUTE PR "Add
optimized_w3", and the arc PR's "The threshold": levers chosen by measurement
on the target part).

Weights and activations are random (torch generator, fixed seed); only their
shapes matter for the timing.  This is a tool, not part of the GEMM path.
"""
from __future__ import annotations

import argparse
import math
import sys

import torch

from . import wq

BF16_ULP_BUDGET = 2
FLOOR_COEF = 1e-3


def _bf16_ord(t):
    """Order-preserving integers for BF16 bit patterns (both zeros -> 0)."""
    b = t.view(torch.int16).to(torch.int32)
    return torch.where(b >= 0, b, -(b & 0x7FFF))


def _inputs(fmt: str, N: int, K: int, M: int, dev: str, seed: int, path: int):
    torch.backends.cuda.matmul.allow_tf32 = False      # the reference is plain FP32
    g = torch.Generator(device="cpu").manual_seed(seed)
    if fmt == "fp8":
        w = torch.randn(N, K, generator=g) * 0.02
        blocks = w.view(N // 128, 128, K // 128, 128)
        amax = blocks.abs().amax(dim=(1, 3))
        scales = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
        q = (blocks / scales[:, None, :, None]).clamp(-448, 448).view(N, K)
        codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
        packed = wq.pack_fp8(codes.to(dev), scales.to(dev))
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev)
        wd = torch.empty(N, K, dtype=torch.float32, device=dev)
        wq.wq_unpack_fp8_block_f32(packed, N, K, wd)
        wd = (wd.view(N // 128, 128, K // 128, 128) * scales.to(dev)[:, None, :, None]).view(N, K)
        call = lambda p, y, ws=None: wq.wq_gemm_fp8_block_path(p, N, K, x, y, M, ws, path)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    else:
        codes = torch.randint(0, 8, (N, K), generator=g, dtype=torch.uint8)
        qmap = torch.sort(torch.randn(8, generator=g)).values.to(torch.float16)
        gs = (torch.rand(N, K // 128, generator=g) * 0.015 + 0.005).to(torch.float16)
        dense = fmt == "lut3d"
        packed = (wq.pack_lut3_dense if dense else wq.pack_lut3)(codes.to(dev), qmap.to(dev), gs.to(dev))
        x = torch.randn(M, K, generator=g).to(torch.float16).to(dev)
        wh = torch.empty(N, K, dtype=torch.float16, device=dev)
        (wq.wq_unpack_lut3_dense if dense else wq.wq_unpack_lut3)(packed, N, K, wh)
        wd = wh.float()
        gemm = wq.wq_gemm_lut3_dense if dense else wq.wq_gemm_lut3
        call = lambda p, y, ws=None: gemm(p, N, K, x, y, M, ws)
        y = torch.empty(M, N, dtype=torch.float16, device=dev)
    ref = x.float() @ wd.t()
    floor = FLOOR_COEF * math.sqrt(K) * x.float().abs().max().item() * wd.abs().max().item()
    return packed, call, y, ref, floor


def _passes(y, ref, floor) -> bool:
    yf = y.float()
    if not torch.isfinite(yf).all():
        return False
    abs_ok = (yf - ref).abs() <= floor
    ulp_ok = (_bf16_ord(yf.to(torch.bfloat16)) - _bf16_ord(ref.to(torch.bfloat16))).abs() <= BF16_ULP_BUDGET
    return bool((abs_ok | ulp_ok).all())


def _time(call, copies, y, calls: int = 100, reps: int = 5) -> float:
    for i in range(10):
        call(copies[i % len(copies)], y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(reps):
        e0.record()
        for i in range(calls):
            call(copies[i % len(copies)], y)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / calls)
    return sorted(out)[reps // 2]


def candidates(fmt: str, gemv: bool = False, kp: int = 1):
    """(nt, sn, split) triples the kernels are built for: sn <= 8, at most 4
    K groups, and at most 8 waves per work-group except the GEMV and one-tile
    LUT groups whose waves hold at most 4 activation pieces per lane
    (sn >= 4), built for 16.  The GEMV always runs one tile per wave."""
    out = []
    for nt in ((1,) if gemv or kp > 1 else (1, 2)):
        for sn in range(1, 9):
            pieces = math.ceil(16 / sn)
            max_split = 16 if (gemv or (fmt in ("lut3", "lut3d") and nt == 1 and pieces <= 4)) else 8
            for sk in (1, 2, 3, 4):
                if sn * sk <= max_split:
                    out.append((nt, sn, sn * sk))
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fmt", choices=("fp8", "lut3", "lut3d"), default="fp8",
                    help="lut3d: the LUT format with codes stored at 3 bits each")
    ap.add_argument("--N", type=int, required=True)
    ap.add_argument("--K", type=int, required=True)
    ap.add_argument("--M", type=int, default=16)
    ap.add_argument("--top", type=int, default=8)
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--path", choices=("mfma", "gemv"), default="mfma", help="FP8 arm to tune (gemv: M <= 4)")
    ap.add_argument("--kparts", default="1",
                    help="comma-separated K-part counts to sweep (> 1: K split across work-groups, with a workspace)")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("tune needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    path = wq.WQ_PATH_GEMV if args.path == "gemv" else wq.WQ_PATH_MFMA
    packed, call, y, ref, floor = _inputs(args.fmt, args.N, args.K, args.M, dev, args.seed, path)
    # rotate copies totalling > the 256 MB Infinity Cache, so calls stream from HBM
    n_copies = min(64, max(2, math.ceil((1 << 30) / packed.numel())))
    copies = [packed] + [packed.clone() for _ in range(n_copies - 1)]
    fmt_id = {"fp8": wq.WQ_FMT_FP8_BLOCK, "lut3": wq.WQ_FMT_LUT3, "lut3d": wq.WQ_FMT_LUT3_DENSE}[args.fmt]
    results, rejected = [], []
    try:
        for kp in (int(v) for v in args.kparts.split(",")):
            wq.wq_set_kparts(kp)
            ws = wq.workspace(fmt_id, args.N, args.K, dev) if kp > 1 else None
            for t in candidates(args.fmt, args.path == "gemv", kp):
                wq.wq_set_tuning(t[0], t[1], t[2], 0)
                y.zero_()
                call(packed, y, ws)
                torch.cuda.synchronize()
                if not _passes(y, ref, floor):
                    rejected.append(t + (kp,))
                    continue
                results.append((_time(lambda p, yy: call(p, yy, ws), copies, y), t + (kp,)))
    finally:
        wq.wq_set_tuning(0, 0, 0, 0)
        wq.wq_set_kparts(0)
    results.sort()
    wb = packed.numel()
    print("%s N=%d K=%d M=%d: %d candidates pass, %d rejected" % (args.fmt, args.N, args.K, args.M,
                                                                 len(results), len(rejected)))
    for us, (nt, sn, split, kp) in results[: args.top]:
        print("  nt=%d sn=%d split=%-2d kp=%-2d %7.2f us  %6.0f GB/s" % (nt, sn, split, kp, us, wb / us / 1e3))
    if rejected:
        print("  rejected:", rejected)
    if results:
        nt, sn, split, kp = results[0][1]
        kind = ("wq::KIND_GEMV_FP8" if args.path == "gemv" else "wq::KIND_MFMA_FP8") if args.fmt == "fp8" \
            else ("wq::KIND_MFMA_LUT3D" if args.fmt == "lut3d" else "wq::KIND_MFMA_LUT")
        print("table row (%s): {%s, %d, %d, %d, %d, %d, %d}," % ("kSplitTable" if kp > 1 else "kTable", kind,
                                                                 args.N, args.K, nt, sn, split, kp))
    return 0 if results else 1


if __name__ == "__main__":
    sys.exit(main())
