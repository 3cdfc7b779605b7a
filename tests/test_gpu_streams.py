"""Calls from several host threads, each on its own stream, at the same time.

The library keeps no per-call state on the host (the compute-unit count is
cached per device with an atomic), so concurrent calls on different streams
must give the same bits as the same calls made one after another.
"""
import threading

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import dev, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu


def test_concurrent_calls_on_separate_streams_match_serial_calls():
    ensure_built()
    dcase = W.decode_case(5000, batch=6, num_qo_heads=32, num_kv_heads=8,
                          seq_lens=[100, 2000, 17, 900, 4096, 1])
    rcase = W.ragged_case(5001, qo_lens=[64, 200, 5], kv_lens=[300, 200, 40], num_qo_heads=16,
                          num_kv_heads=4)
    kv = dcase.kv
    dq, kp, vp = dev(dcase.q), dev(kv.k_pool), dev(kv.v_pool)
    dargs = (dev(kv.page_indptr), dev(kv.page_indices), dev(kv.seq_lens))
    rq, rk, rv = dev(rcase.q), dev(rcase.k), dev(rcase.v)
    ri, rki = dev(rcase.qo_indptr), dev(rcase.kv_indptr)
    nthreads, reps = 4, 8
    torch.cuda.synchronize()  # inputs are in place before other streams read them

    def work(outs, stream):
        with torch.cuda.stream(stream):
            for r in range(reps):
                od, orr = outs[r]
                assert oxa.oxa_paged_decode(dq, kp, vp, *dargs, od, max_seq_len=4096,
                                            sm_scale=dcase.sm_scale, num_kv_heads=8,
                                            stream=stream) == oxa.OXA_OK
                assert oxa.oxa_ragged_prefill(rq, rk, rv, ri, rki, orr, max_qo_len=200,
                                              max_kv_len=300, sm_scale=rcase.sm_scale,
                                              causal=True, stream=stream) == oxa.OXA_OK

    def fresh():
        return [[(torch.empty_like(dq), torch.empty_like(rq)) for _ in range(reps)]
                for _ in range(nthreads)]

    note("serial reference calls")
    serial = fresh()
    s0 = torch.cuda.Stream()
    for t in range(nthreads):
        work(serial[t], s0)
    torch.cuda.synchronize()

    note("concurrent calls from 4 threads on 4 streams")
    conc = fresh()
    streams = [torch.cuda.Stream() for _ in range(nthreads)]
    errors = []

    def run(t):
        try:
            work(conc[t], streams[t])
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(t,)) for t in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(nthreads):
        for r in range(reps):
            assert torch.equal(conc[t][r][0], serial[t][r][0]), f"decode thread {t} rep {r}"
            assert torch.equal(conc[t][r][1], serial[t][r][1]), f"prefill thread {t} rep {r}"
    # and every repetition equals the first (the kernels are deterministic)
    for t in range(nthreads):
        for r in range(reps):
            assert torch.equal(conc[t][r][0], serial[0][0][0])
            assert torch.equal(conc[t][r][1], serial[0][0][1])
