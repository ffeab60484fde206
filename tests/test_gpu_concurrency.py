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
    jobs = _jobs()
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
                for r in range(ROUNDS):
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
