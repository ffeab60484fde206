"""Calls from several host threads at once, each on its own HIP stream with
its own workspace and outputs (the header's thread-safety rule): FP8 with K
parts, both LUT layouts and the W8A8 tier over several shapes and M, so the
threads also race on the plan cache.  Every result must equal the same call
made serially, bit for bit (the results are deterministic)."""
import threading

import numpy as np
import pytest
import torch

import synth
import gpu_util as U

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 12


def _jobs():
    """(name, make_outputs, call(outs, stream)) for each kind of call."""
    wq = U.wqmod()
    jobs = []
    for (N, K, M) in ((1024, 2048, 16), (640, 2560, 5), (512, 1152, 32)):
        codes, scales = synth.fp8_weights(N, K, 2000 + N)
        packed = U.pack_fp8(codes, scales)
        x = U.t_u16(synth.x_bf16(M, K, 2001 + M), torch.bfloat16)
        nb = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8_BLOCK, M, N, K)

        def make(N=N, M=M, nb=nb):
            return {"y": torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV),
                    "ws": torch.empty(max(nb, 16), dtype=torch.uint8, device=U.DEV)}

        def call(o, s, packed=packed, N=N, K=K, M=M, x=x, nb=nb):
            wq.wq_gemm_fp8_block(packed, N, K, x, o["y"], M, o["ws"] if nb else None, stream=s)
        jobs.append(("fp8-%dx%d-M%d" % (N, K, M), make, call))
    for dense in (False, True):
        N, K, M = 528, 4096, 20
        c, q, g = synth.lut3_weights(N, K, 2010)
        packed = U.pack_lut3(c, q, g, dense=dense)
        x = U.t_u16(synth.x_f16(M, K, 2011), torch.float16)
        gemm = wq.wq_gemm_lut3_dense if dense else wq.wq_gemm_lut3

        fmt = wq.WQ_FMT_LUT3_DENSE if dense else wq.WQ_FMT_LUT3
        nb = wq.wq_gemm_workspace_bytes(fmt, M, N, K)

        def make(N=N, M=M, nb=nb):
            return {"y": torch.empty((M, N), dtype=torch.float16, device=U.DEV),
                    "ws": torch.empty(max(nb, 16), dtype=torch.uint8, device=U.DEV)}

        def call(o, s, packed=packed, N=N, K=K, M=M, x=x, gemm=gemm, nb=nb):
            gemm(packed, N, K, x, o["y"], M, o["ws"] if nb else None, stream=s)
        jobs.append(("lut3%s" % ("d" if dense else ""), make, call))
    N, K, M = 640, 2048, 48
    codes, scales = synth.fp8_weights(N, K, 2020)
    packed = U.pack_fp8(codes, scales)
    x = U.t_u16(synth.x_bf16(M, K, 2021), torch.bfloat16)
    nb = wq.wq_w8a8_workspace_bytes(M, N, K)

    def make_w8(N=N, K=K, M=M, nb=nb):
        return {"y": torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV),
                "xq": torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=U.DEV),
                "ws": torch.empty(max(nb, 16), dtype=torch.uint8, device=U.DEV)}

    def call_w8(o, s, packed=packed, N=N, K=K, M=M, x=x, nb=nb):
        wq.wq_quantize_x_fp8(x, M, K, o["xq"], stream=s)
        wq.wq_gemm_fp8_w8a8(packed, N, K, o["xq"], M, o["y"], o["ws"] if nb else None, stream=s)
    jobs.append(("w8a8", make_w8, call_w8))
    return jobs


@pytest.fixture
def three_parts():
    """K split in 3 parts across work-groups wherever a call passes a
    workspace (clamped where a part would get no K block)."""
    U.wqmod().wq_set_kparts(3)
    yield
    U.wqmod().wq_set_kparts(0)


def test_concurrent_threads_and_streams_match_serial(three_parts):
    U.note("concurrency: %d threads x %d rounds" % (THREADS, ROUNDS))
    _run_concurrently(_jobs(), ROUNDS)


def _w8a8_job(N, K, M, seed, ws):
    wq = U.wqmod()
    codes, scales = synth.fp8_weights(N, K, seed)
    packed = U.pack_fp8(codes, scales)
    x = U.t_u16(synth.x_bf16(M, K, seed + 1), torch.bfloat16)
    nb = wq.wq_w8a8_workspace_bytes(M, N, K) if ws else 0

    def make():
        return {"y": torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV),
                "xq": torch.empty(wq.wq_x_fp8_packed_bytes(M, K), dtype=torch.uint8, device=U.DEV),
                "ws": torch.empty(max(nb, 16), dtype=torch.uint8, device=U.DEV)}

    def call(o, s):
        wq.wq_quantize_x_fp8(x, M, K, o["xq"], stream=s)
        wq.wq_gemm_fp8_w8a8(packed, N, K, o["xq"], M, o["y"], o["ws"] if nb else None, stream=s)
    return ("w8a8-%dx%d-M%d-%s" % (N, K, M, "ws" if ws else "nows"), make, call)


def test_concurrent_w8a8_column_bands_match_serial():
    """W8A8 calls that run in two column bands (on 256 CUs: a leading band of
    whole rounds, then the rest of the columns as a second launch, with K
    split there when a workspace is passed), from four threads on their own
    streams beside one-band calls: every result equals the serial call."""
    wq = U.wqmod()
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    N, K, M = 16640, 4096, 897
    U.note("concurrency: W8A8 bands %s / %s" % (wq.wq_query_w8a8_plan(M, N, K, cu, True),
                                                wq.wq_query_w8a8_plan(M, N, K, cu, False)))
    if cu == 256:
        assert wq.wq_query_w8a8_plan(M, N, K, cu, True)["tail"] == (128, 128, 2)
        assert wq.wq_query_w8a8_plan(M, N, K, cu, False)["tail"] == (128, 128, 1)
    jobs = [_w8a8_job(N, K, M, 2030, True), _w8a8_job(N, K, M, 2030, False), _w8a8_job(640, 2048, 300, 2040, True)]
    _run_concurrently(jobs, 4)


def _run_concurrently(jobs, rounds):
    ref = {}
    for name, make, call in jobs:                 # serial reference on the current stream
        o = make()
        call(o, None)
        torch.cuda.synchronize()
        ref[name] = o["y"].clone()
    errors = []
    results = [dict() for _ in range(THREADS)]

    def worker(t):
        try:
            s = torch.cuda.Stream()
            outs = {name: make() for name, make, _ in jobs}
            with torch.cuda.stream(s):
                for r in range(rounds):
                    order = jobs if (r + t) % 2 == 0 else list(reversed(jobs))
                    for name, _, call in order:
                        outs[name]["y"].fill_(float("nan"))
                        call(outs[name], s)
            s.synchronize()
            results[t] = {name: o["y"].clone() for name, o in outs.items()}
        except Exception as e:                    # reported after the join
            errors.append("thread %d: %r" % (t, e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
    for t in range(THREADS):
        for name, y in results[t].items():
            assert torch.equal(y.view(torch.int16), ref[name].view(torch.int16)), (t, name)
