#!/usr/bin/env python3
"""Benchmark of the decode-phase weight-only-quantized GEMM on one MI355X.

A step is one call of the hot path (dispatch, weight stream, activation staging,
dequant, matrix-core inner product, split-K scheduling, epilogue) on one batch:
by default the FP8 block-scaled FFN gate/up projection, N=17408, K=5120, M=16,
BF16 activations.  Inputs are synthetic and seeded (synth/), already resident in
HBM before timing starts.  Each step reads a different copy of the packed
weight matrix, and the copies together exceed the 256 MB Infinity Cache, so the
weight bytes of every step come from HBM.

Reported value: weight-stream GB/s = (packed code bytes + scale bytes) per step
divided by the time per step (the pages count stored weight bytes: one byte an
FP8 code, half a byte a nibble-packed 3-bit code, 3/8 a dense one, plus the
scales).  The JSON line also carries the dominant kernel's roofline (bytes
per launch over the mean launch duration, from HIP events on the library's
stream), the CPU oracle timed on the host as a baseline (whose output also
grades the timed steps' output element by element: "parity" in that object),
and an "extra" block
with the other M=16 target (3-bit LUT 28672 x 8192, both storage layouts), the
FFN down projection at M = 16 and 32 and gate/up at M = 1 and 8 (--no-extra
skips it; --all times every workload, M and the W8A8 tier).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight-stream GB/s (% of HBM peak) for quantized GEMM at M=1/8/16/32"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
ROTATE_TARGET_BYTES = 1 << 30
WARM_SECONDS = 0.2
SPREAD_WINDOWS = 9


def weight_bytes(fmt: str, N: int, K: int) -> int:
    """Packed bytes a call streams: codes + scales (+ the LUT map)."""
    if fmt == "fp8":
        return N * K + 4 * (N // 128) * (K // 128)
    code_bytes = N * K * 3 // 8 if fmt == "lut3d" else N * K // 2     # 3 bits or one nibble a code
    return code_bytes + 16 * N * ((K // 128 + 7) // 8) + 16


def algorithmic_bytes(fmt: str, N: int, K: int, M: int) -> int:
    """Bytes a launch must move: weight stream + activations in + outputs out."""
    return weight_bytes(fmt, N, K) + 2 * M * K + 2 * M * N


def kernel_src_sha() -> str:
    """Hash of the library's sources with comments and layout removed, so a
    change to a comment does not orphan counter data taken on the same code."""
    h = hashlib.sha256()
    for f in ("wq_kernels.hip", "wq_w8a8.hip", "wq_device.hpp", "wq_internal.h", "wq_api.cpp"):
        with open(os.path.join(ROOT, "weight_only_quantized_fp8_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def sysfs_gpu_state(node: str) -> dict:
    """Current shader clock level (the DPM table line marked '*') and hwmon
    temperatures and clocks of the PCI device node `node`; {} where absent."""
    import glob
    st = {}
    try:
        if os.path.exists(node + "/pp_dpm_sclk"):
            with open(node + "/pp_dpm_sclk") as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        st["sclk_level"] = line.split(":", 1)[1].strip(" *\n")
        for path in sorted(glob.glob(node + "/hwmon/hwmon*/temp*_input") + glob.glob(node + "/hwmon/hwmon*/freq*_input")):
            label = path[:-len("_input")] + "_label"
            name = open(label).read().strip() if os.path.exists(label) else os.path.basename(path)[:-len("_input")]
            v = int(open(path).read())
            if os.path.basename(path).startswith("temp"):
                st["temp_%s_C" % name] = v / 1000.0          # millidegrees
            else:
                st["%s_MHz" % name] = round(v / 1e6)          # Hz
    except (OSError, ValueError):
        pass
    return st


def gpu_state() -> dict:
    """sysfs_gpu_state of cuda:0 (found by its PCI address).  Reads files only:
    no tool is started."""
    try:
        import torch
        pr = torch.cuda.get_device_properties(0)
    except Exception:
        return {}
    return sysfs_gpu_state("/sys/bus/pci/devices/%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id,
                                                                      pr.pci_device_id))


def load_traffic(workload_key: str):
    """HBM traffic per launch measured with rocprofv3 PMC counters for this kernel
    source (profiles/traffic.json); None when absent or the kernel changed."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(workload_key)
        if not e or e.get("kernel_src_sha") != kernel_src_sha():
            return None
        return float(e["hbm_bytes_per_launch"])
    except Exception:
        return None


class Workload:
    def __init__(self, name: str, M: int, copies: int | None = None):
        import numpy as np
        import torch
        import synth
        from weight_only_quantized_fp8_amd import wq

        self.name, self.M = name, M
        self.fmt, self.N, self.K, _ = synth.CONFIGS[name]
        N, K = self.N, self.K
        seed = synth.SEEDS[name]
        dev = "cuda:0"
        self.wbytes = weight_bytes(self.fmt, N, K)
        self.abytes = algorithmic_bytes(self.fmt, N, K, M)
        if copies is None:
            copies = max(2, math.ceil(ROTATE_TARGET_BYTES / self.wbytes))
        self.copies = copies
        if self.fmt == "fp8":
            codes, scales = synth.fp8_weights(N, K, seed)
            p0 = wq.pack_fp8(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
            x = synth.x_bf16(M, K, seed + 100)
            self.x = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            self.ws = wq.workspace(wq.WQ_FMT_FP8_BLOCK, N, K, dev)
            self._call = lambda p: wq.wq_gemm_fp8_block(p, N, K, self.x, self.y, M, self.ws)
        else:
            dense = self.fmt == "lut3d"
            codes, qmap, g = synth.lut3_weights(N, K, seed)
            t16 = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16)
            pack = wq.pack_lut3_dense if dense else wq.pack_lut3
            p0 = pack(torch.from_numpy(codes).to(dev), t16(qmap), t16(g))
            del codes
            x = synth.x_f16(M, K, seed + 100)
            self.x = t16(x)
            self.y = torch.empty((M, N), dtype=torch.float16, device=dev)
            self.ws = wq.workspace(wq.WQ_FMT_LUT3_DENSE if dense else wq.WQ_FMT_LUT3, N, K, dev)
            gemm = wq.wq_gemm_lut3_dense if dense else wq.wq_gemm_lut3
            self._call = lambda p: gemm(p, N, K, self.x, self.y, M, self.ws)
        # K parts the shape's workspace plan splits K into (1: no workspace needed)
        self.k_parts = max(1, self.ws.numel() // (32 * N * 4))
        self.packed = [p0] + [p0.clone() for _ in range(copies - 1)]
        torch.cuda.synchronize()
        self.i = 0

    def step(self):
        self._call(self.packed[self.i % self.copies])
        self.i += 1

    def launches_per_step(self) -> int:
        # passes over the weights per step: the per-shape plans run one tile
        # per wave, which serves M = 17..32 in a single pass (both 16-row
        # halves share each dequantised operand); a K split across
        # work-groups adds a small kernel that sums the parts, not a pass
        return 1


def time_workload(w: Workload, steps: int, warmup: int, use_graph: bool = True):
    """Time `steps` back-to-back steps between two HIP events on the stream the
    library launches on.  With use_graph the steps are captured once into a HIP
    graph and replayed, so the host's per-call launch cost (Python, ctypes,
    hipLaunchKernel) does not sit between the kernels; the graph's output is
    checked bit for bit against an eager call first."""
    import torch
    for _ in range(min(warmup, 20)):
        w.step()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        w.i = 0
        w.step()                                   # eager reference on copy 0
        torch.cuda.synchronize()
        ref = w.y.clone()
        w.y.zero_()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            graph = torch.cuda.CUDAGraph()
            w.i = 0
            with torch.cuda.graph(graph, stream=s):
                for _ in range(steps):
                    w.step()
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(2):                       # replays agree with the eager result
            w.y.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            # the last captured step used copy (steps-1) % copies, identical bytes to copy 0
            if not torch.equal(w.y.view(torch.int16), ref.view(torch.int16)):
                raise RuntimeError("graph replay %d differs from the eager result" % rep)
    # The rest of the warm-up: at least `warmup` steps in all and at least
    # WARM_SECONDS of back-to-back work, so the part's clock has settled to
    # its sustained value before the timed steps (it ramps over the first
    # milliseconds of load).
    done, t_warm = min(warmup, 20), time.perf_counter()
    while done < warmup or time.perf_counter() - t_warm < WARM_SECONDS:
        if graph is not None:
            graph.replay()
            done += steps
        else:
            for _ in range(100):
                w.step()
            done += 100
        torch.cuda.synchronize()          # keeps the host's clock on the GPU's work
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    t0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(steps):
            w.step()
    t1.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    total_ms = t0.elapsed_time(t1)
    # Spread: SPREAD_WINDOWS more windows of the same steps after the timed
    # one (reported beside it; the value is the timed window alone).
    windows = [total_ms / steps]
    if graph is not None:
        for _ in range(SPREAD_WINDOWS):
            t0.record(stream)
            graph.replay()
            t1.record(stream)
            torch.cuda.synchronize()
            windows.append(t0.elapsed_time(t1) / steps)
    q = sorted(windows)
    pick = lambda f: q[min(len(q) - 1, int(round(f * (len(q) - 1))))]
    return {
        "ms_per_step": total_ms / steps,
        "host_ms_per_step": host_s * 1e3 / steps,
        "launch_ms_mean": total_ms / steps / w.launches_per_step(),
        "graph": graph is not None,
        "windows_us": {"n": len(q), "p10": round(pick(0.1) * 1e3, 3), "median": round(pick(0.5) * 1e3, 3),
                       "p90": round(pick(0.9) * 1e3, 3)},
    }


FP8_MFMA_PEAK_TFLOPS = 5000.0

# Workloads a default run times beside the headline one, by the same method
# (HIP graph of the steps, weight copies rotated beyond the Infinity Cache):
# the other M=16 target (3-bit LUT 28672 x 8192, both storage layouts), the
# FFN down projection at M = 16 and 32, and gate/up at M = 1 and 8.
DEFAULT_EXTRA = [("lut3", 16), ("lut3d", 16), ("down", 16), ("down", 32), ("gate_up", 1), ("gate_up", 8)]


def time_extra(name: str, M: int, steps: int, warmup: int, eager: bool) -> dict:
    """One more workload timed like the headline one; its line of the extra block."""
    import synth
    import torch
    fmt, N, K, _ = synth.CONFIGS[name]
    print("bench: %s M=%d" % (name, M), file=sys.stderr, flush=True)
    wk = Workload(name, M)
    rk = time_workload(wk, steps, warmup, use_graph=not eager)
    state = gpu_state()
    gbs = wk.wbytes * wk.launches_per_step() / (rk["ms_per_step"] * 1e-3) / 1e9
    e = {"us_per_call": round(rk["ms_per_step"] * 1e3, 2),
         "windows_us": rk["windows_us"],
         "stream_GBps": round(gbs, 1), "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
         "roofline_frac": round(wk.abytes / (rk["launch_ms_mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "passes": wk.launches_per_step(), "k_parts": wk.k_parts, "sclk_after": state.get("sclk_level")}
    if fmt in ("lut3", "lut3d"):
        # 3 bits of information per code, plus the group scales and the map
        info = N * K * 3 // 8 + 2 * N * (K // 128) + 16
        e["info_GBps"] = round(info / (rk["ms_per_step"] * 1e-3) / 1e9, 1)
    del wk
    torch.cuda.empty_cache()
    return e


def time_w8a8(name: str, M: int, steps: int = 20, copies: int = 4) -> dict:
    """The W8A8 tier on an FFN shape at a prefill batch: one step quantises the
    BF16 activations (wq_quantize_x_fp8) and runs wq_gemm_fp8_w8a8 on a packed
    FP8 weight matrix; `copies` weight copies (more than the 256 MB Infinity
    Cache together) rotate over the steps.  The steps are replayed from a HIP
    graph, timed with HIP events; the two kernels are also timed alone."""
    import numpy as np
    import torch
    import synth
    from weight_only_quantized_fp8_amd import wq
    fmt, N, K, _ = synth.CONFIGS[name]
    dev = "cuda:0"
    codes, scales = synth.fp8_weights(N, K, synth.SEEDS[name])
    p0 = wq.pack_fp8(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    del codes
    packed = [p0] + [p0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.x_bf16(M, K, synth.SEEDS[name] + 100).view(np.int16)).to(dev).view(torch.bfloat16)
    xq = torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # the workspace lets a thin grid split K across work-groups (FFN down at small M)
    ws_bytes = wq.wq_w8a8_workspace_bytes(M, N, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    plan = wq.wq_query_w8a8_plan(M, N, K, cu, ws is not None)
    k_parts = plan["kparts"]
    tile = "%dx%d%s" % (plan["tile"] + (" streaming" if plan["streaming"] else "",))
    if plan["tail"]:   # two column bands: the rest of the columns on their own plan
        tile += ", columns %d-%d on %dx%d in %d parts" % ((plan["band"], N - 1) + plan["tail"])

    def step(i):
        wq.wq_quantize_x_fp8(x, M, K, xq)
        wq.wq_gemm_fp8_w8a8(packed[i % copies], N, K, xq, M, y, ws)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record()
    g.replay()
    ev[1].record()
    for i in range(steps):
        wq.wq_quantize_x_fp8(x, M, K, xq)
    ev[2].record()
    ev[3].record()
    for i in range(steps):
        wq.wq_gemm_fp8_w8a8(packed[i % copies], N, K, xq, M, y, ws)
    ev[4].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    q_us = ev[1].elapsed_time(ev[2]) * 1e3 / steps
    g_us = ev[3].elapsed_time(ev[4]) * 1e3 / steps
    tf = 2.0 * M * N * K / (g_us * 1e-6) / 1e12
    del packed, g
    torch.cuda.empty_cache()
    return {"us_per_call": round(us, 2), "quantize_us": round(q_us, 2), "gemm_us": round(g_us, 2),
            "gemm_TFLOPs": round(tf, 1), "pct_of_fp8_mfma_peak": round(100 * tf / FP8_MFMA_PEAK_TFLOPS, 1),
            "k_parts": k_parts, "tile": tile}


def graph_time_us(step, steps: int = 100, windows: int = 9) -> dict:
    """Median (and p10/p90) microseconds per step of `step(i)` over `windows`
    replays of a HIP graph holding `steps` calls, after a settling warm-up."""
    import torch
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    t_end = time.perf_counter() + WARM_SECONDS
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    v = []
    for _ in range(windows):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        v.append(e0.elapsed_time(e1) * 1e3 / steps)
    v.sort()
    pick = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
    del g
    return {"median": round(pick(0.5), 2), "p10": round(pick(0.1), 2), "p90": round(pick(0.9), 2)}


def crossover() -> dict:
    """The arms of the decode ladder on one binary (the arc PR's "The threshold":
    every arm timed on the same build, the crossover taken from the data).
    (1) FP8 strict-order GEMV against the 16-row MFMA tile at M = 1..4 on the
    FFN and attention shapes; (2) the W8A8 tier (quantise + FP8 x FP8 GEMM,
    with its workspace) against the decode tile run as 32-row calls
    (ceil(M/32) calls on consecutive row blocks) at M = 16 .. 128.  Weight
    copies rotate beyond the Infinity Cache in both."""
    import numpy as np
    import torch
    import synth
    from weight_only_quantized_fp8_amd import wq
    dev = "cuda:0"
    out = {"gemv_vs_mfma": {}, "w8a8_vs_decode": {}}
    for name in ("gate_up", "down", "attn_q", "attn_o", "attn_k"):
        fmt, N, K, _ = synth.CONFIGS[name]
        codes, scales = synth.fp8_weights(N, K, synth.SEEDS[name])
        p0 = wq.pack_fp8(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
        del codes
        copies = max(2, math.ceil(ROTATE_TARGET_BYTES / p0.numel()))
        packed = [p0] + [p0.clone() for _ in range(copies - 1)]
        ws = wq.workspace(wq.WQ_FMT_FP8_BLOCK, N, K, dev)
        ws = ws if ws.numel() else None
        row = {}
        for M in (1, 2, 3, 4):
            x = torch.from_numpy(synth.x_bf16(M, K, synth.SEEDS[name] + 100).view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for path, tag in ((wq.WQ_PATH_GEMV, "gemv"), (wq.WQ_PATH_MFMA, "mfma")):
                print("bench: crossover %s M=%d %s" % (name, M, tag), file=sys.stderr, flush=True)
                st = lambda i, x=x, y=y, path=path: wq.wq_gemm_fp8_block_path(packed[i % copies], N, K, x, y, M, ws,
                                                                              path)
                row["M%d_%s_us" % (M, tag)] = graph_time_us(st)["median"]
        out["gemv_vs_mfma"][name] = row
        if name in ("gate_up", "down"):
            r2 = {}
            for M in (16, 32, 33, 40, 48, 64, 96, 128):
                x = torch.from_numpy(synth.x_bf16(M, K, synth.SEEDS[name] + 100).view(np.int16)).to(dev).view(
                    torch.bfloat16)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                print("bench: crossover %s M=%d decode vs w8a8" % (name, M), file=sys.stderr, flush=True)

                def dec(i, x=x, y=y, M=M):
                    for r0 in range(0, M, 32):
                        wq.wq_gemm_fp8_block(packed[i % copies], N, K, x[r0:r0 + 32], y[r0:r0 + 32], min(32, M - r0), ws)
                xq = torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=dev)
                nb = wq.wq_w8a8_workspace_bytes(M, N, K)
                w8ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None

                def w8(i, x=x, y=y, M=M, xq=xq, w8ws=w8ws):
                    wq.wq_quantize_x_fp8(x, M, K, xq)
                    wq.wq_gemm_fp8_w8a8(packed[i % copies], N, K, xq, M, y, w8ws)
                d_us, w_us = graph_time_us(dec)["median"], graph_time_us(w8)["median"]
                r2["M%d" % M] = {"decode_us": d_us, "decode_calls": (M + 31) // 32, "w8a8_us": w_us,
                                 "faster": "decode" if d_us < w_us else "w8a8"}
            out["w8a8_vs_decode"][name] = r2
        del packed, p0
        torch.cuda.empty_cache()
    return out


def cpu_baseline(name: str, M: int, min_seconds: float = 10.0, max_reps: int = 500, gpu_bits=None):
    """The oracle as it stands, on the host cores, over the whole workload (all
    outputs), repeated until about min_seconds of CPU wall time (at least 3
    passes); the median pass counts.  With gpu_bits (the GPU's output of the
    same seeded workload as BF16/FP16 bits [M, N]) the oracle's output also
    grades it, element by element under the library's rule (within 2 BF16 ULP
    or the absolute floor): the receipt comes back as "parity"."""
    import numpy as np
    import oracle
    from oracle import compare
    import synth
    fmt, N, K, _ = synth.CONFIGS[name]
    seed = synth.SEEDS[name]
    threads = oracle.default_threads()
    if fmt == "fp8":
        codes, scales = synth.fp8_weights(N, K, seed)
        x = synth.x_bf16(M, K, seed + 100)
        run = lambda: oracle.gemm_fp8(x, codes, scales, nthreads=threads)
    else:
        codes, qmap, g = synth.lut3_weights(N, K, seed)
        x = synth.x_f16(M, K, seed + 100)
        run = lambda: oracle.gemm_lut3(x, codes, qmap, g, nthreads=threads)
    times = []
    start = time.perf_counter()
    y64 = None
    while len(times) < max_reps and (time.perf_counter() - start < min_seconds or len(times) < 3):
        t0 = time.perf_counter()
        y64 = run()
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    res = {"value": weight_bytes(fmt, N, K) / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "whole %s workload N=%d K=%d M=%d, all %d outputs; median of %d passes "
                     "(%.1f s of CPU work in all), %.3f s each"
                     % (name, N, K, M, M * N, len(times), sum(times), dt),
           "seconds": dt}
    if gpu_bits is not None:
        # floor inputs: max |x| and max |dequantised weight|, the weights in row chunks
        if fmt == "fp8":
            mx = float(np.abs(oracle.bf16_value(x)).max())
            mw = max(float(np.nanmax(np.abs(oracle.dequant_fp8(codes[r:r + 2048], scales[r // 128:(r + 2048) // 128]))))
                     for r in range(0, N, 2048))
        else:
            mx = float(np.abs(oracle.f16_value(x)).max())
            mw = max(float(np.abs(oracle.dequant_lut3(codes[r:r + 2048], qmap, g[r:r + 2048])).max())
                     for r in range(0, N, 2048))
        rc = compare.grade(gpu_bits, y64, compare.abs_floor(K, mx, mw), "bf16" if fmt == "fp8" else "f16")
        res["parity"] = {"ok": rc.ok, "n": rc.n, "fail": rc.n_fail, "max_ulp": rc.max_ulp,
                         "over_2ulp": rc.n_over_budget, "max_err_over_floor": round(rc.max_err_over_floor, 4),
                         "rel_rms": round(rc.rel_rms, 6), "sign_flips": rc.sign_flips}
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="gate_up")
    ap.add_argument("--M", type=int, default=16)
    ap.add_argument("--all", action="store_true", help="also time every other workload and M, and the W8A8 tier")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the headline workload (skip the default extra block)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true", help="launch each step from Python instead of a HIP graph")
    ap.add_argument("--crossover", action="store_true",
                    help="time the ladder's arms on one binary (GEMV vs MFMA at M=1..4, W8A8 vs the decode tile at "
                         "M=16..128) and print that table as one JSON line")
    ap.add_argument("--w8a8", action="store_true",
                    help="time only the W8A8 tier (quantise + FP8 x FP8 GEMM) on --config at --M and print its line")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (its kernels are sized for "
              "one GPU's share of a projection). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    import synth
    if args.crossover:
        print(json.dumps({"crossover": crossover()}), flush=True)
        return 0
    if args.w8a8:
        fmt, N, K, _ = synth.CONFIGS[args.config]
        if fmt != "fp8":
            print("--w8a8 needs an FP8 workload", file=sys.stderr)
            return 2
        r = time_w8a8(args.config, args.M, steps=args.steps)
        print(json.dumps({"metric": "W8A8 GEMM TFLOP/s (quantise + FP8 x FP8 GEMM per step)",
                          "value": r["gemm_TFLOPs"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                          "higher_is_better": True, "dtype": "fp8", "data": "synthetic",
                          "config": {"workload": "%s w8a8 N=%d K=%d M=%d" % (args.config, N, K, args.M)},
                          "roofline": {"bound": "mfma", "achieved": r["gemm_TFLOPs"],
                                       "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(r["gemm_TFLOPs"] / FP8_MFMA_PEAK_TFLOPS, 4)},
                          "timing": r}), flush=True)
        return 0
    print("bench: preparing %s M=%d" % (args.config, args.M), file=sys.stderr, flush=True)
    w = Workload(args.config, args.M)
    state_before = gpu_state()
    r = time_workload(w, args.steps, args.warmup, use_graph=not args.eager)
    state_after = gpu_state()
    # the timed steps' output (bit-identical to the eager reference: checked
    # by time_workload), graded against the oracle in the CPU-baseline leg
    import numpy as np
    gpu_bits = w.y.view(torch.int16).cpu().numpy().view(np.uint16)
    value = w.wbytes / (r["ms_per_step"] * 1e-3) / 1e9
    achieved = w.abytes / (r["launch_ms_mean"] * 1e-3) / 1e9
    key = "%s_M%d" % (args.config, args.M)
    traffic = load_traffic(key)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.fmt == "fp8" else "f16",
        "data": "synthetic",
        "config": {"workload": "%s %s N=%d K=%d M=%d" % (args.config, w.fmt, w.N, w.K, args.M),
                   "format": {"fp8": "fp8_e4m3_block128x128", "lut3": "lut3_group128",
                              "lut3d": "lut3_dense_group128"}[w.fmt],
                   "N": w.N, "K": w.K, "M": args.M, "weight_bytes_per_step": w.wbytes,
                   "weight_copies_rotated": w.copies, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": w.abytes,
                     "launch_us_mean": round(r["launch_ms_mean"] * 1e3, 3)},
        "timing": {"us_per_step": round(r["ms_per_step"] * 1e3, 3),
                   "host_us_per_step": round(r["host_ms_per_step"] * 1e3, 3),
                   "hip_graph": r["graph"],
                   "method": "HIP events around %d back-to-back steps on the library's stream" % args.steps,
                   "windows_us_per_step": r["windows_us"],
                   "gpu_before": state_before, "gpu_after": state_after},
    }
    del w
    torch.cuda.empty_cache()

    extra_list = []
    if args.all:
        extra_list = [(name, M) for name, (fmt, N, K, Ms) in synth.CONFIGS.items() if name != "tiny" for M in Ms]
    elif not args.no_extra:
        extra_list = list(DEFAULT_EXTRA)
    extra_list = [(n, m) for n, m in extra_list if not (n == args.config and m == args.M)]
    if extra_list or args.all:
        extra = {}
        for name, M in extra_list:
            extra["%s_M%d" % (name, M)] = time_extra(name, M, args.steps, args.warmup, args.eager)
        if args.all:
            for name in ("gate_up", "down"):
                for M in (64, 128, 256, 512, 2048, 4096):
                    print("bench: w8a8 %s M=%d" % (name, M), file=sys.stderr, flush=True)
                    extra["w8a8_%s_M%d" % (name, M)] = time_w8a8(name, M)
        out["extra"] = extra

    if not args.no_cpu:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb = cpu_baseline(args.config, args.M, gpu_bits=gpu_bits)
        out["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cb.items()
                               if k != "seconds"}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
