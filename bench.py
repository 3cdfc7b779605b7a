"""Benchmark: paged-decode HBM GB/s + causal-prefill TFLOPS on one MI355X.

One JSON line on stdout.  The timed step is one paged batch decode over the
batch-32 GQA4 workload (32 q / 8 kv heads, head dim 128, page size 16,
seq_lens uniform in [512, 4096], pages shuffled in a shared NHD pool, seed
1002); `value` is its algorithmic HBM bytes / measured step time.  Every step
reads a different copy of the KV pool (copies rotate, > 1 GiB apart), so each
step streams its KV from HBM rather than from the 256 MB last-level cache.

The same run also measures, as extra fields, the long-context causal prefill
(RoPE + exclusive paged append of 2 x 16384 tokens, then paged causal prefill
over those pages; TFLOPS against the bf16 matrix-core peak), the ragged GQA4
prefill, the long MQA split-K decode and the tiny MHA decode.  Kernel-level
durations come from HIP events on the launching stream; the oracle's CPU
throughput on the decode workload is reported as `cpu_baseline`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only ROW]
       [--no-cpu-baseline] [--decode-partitions P]
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, TFLOP/s
ROWS = ("decode", "decode_mha", "decode_mqa", "decode_skewed", "prefill_ragged", "append",
        "prefill_paged", "pages_shapes", "merge", "rope", "copy")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- helpers

def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


class LaunchTimer:
    """Per-launch HIP event pairs on the given stream plus a whole-region pair."""

    def __init__(self, torch, stream, n):
        self.torch = torch
        self.stream = stream
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)]

    def run(self, fn, n):
        for i in range(n):
            a, b = self.pairs[i]
            a.record(self.stream)
            fn(i)
            b.record(self.stream)

    def launch_ms(self, n):
        self.torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in self.pairs[:n]])


def warm_clock(torch, fn, seconds=0.3):
    """Call fn until `seconds` of wall time have passed: the GPU's clock ramps
    up under sustained load, and the extra rows are timed at its steady state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def cold_launch_samples(torch, stream, fn, n, scratch):
    """n launches of fn, each between its own event pair, with a 1 GiB scratch
    write before each (outside the pair) so the launch finds caches cold.
    Returns the per-launch durations in ms."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for i, (a, b) in enumerate(pairs):
        scratch.fill_(i & 0xff)
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in pairs])


def decode_bytes(case):
    """Algorithmic HBM bytes of one paged decode: K+V rows of every token of every
    sequence and kv head, q in, o out, and the page table read."""
    kv = case.kv
    hkv = kv.num_kv_heads
    B, hq, d = case.q.shape
    tokens = int(np.sum(kv.seq_lens.astype(np.int64)))
    pages = int(np.sum((kv.seq_lens.astype(np.int64) + 15) // 16))
    return tokens * hkv * d * 2 * 2 + 2 * B * hq * d * 2 + pages * 4 + (2 * B + 1) * 4


def causal_flops(qo_lens, kv_lens, hq, d=128):
    """Matrix flops of causal attention (QK^T and PV) over the visible pairs
    (bottom-right alignment): 4 * d * hq per (query, key) pair."""
    pairs = 0
    for q, k in zip(qo_lens, kv_lens):
        q, k = int(q), int(k)
        pairs += q * (k - q + 1) + q * (q - 1) // 2
    return 4 * d * hq * pairs


def source_hash(name):
    path = os.path.join(ROOT, "paged_attention_02_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def profiled_traffic(kernel_file, profile_name):
    """HBM bytes per launch recorded from rocprofv3 counters, if the kernel source
    has not changed since (the summary records the source hash)."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source sha256\[:16\]:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(kernel_file):
        return None
    return float(m_bytes.group(1))


# ----------------------------------------------------------------------------- rows

def bench_decode(torch, oxa, W, case, steps, warmup, scratch, copies_bytes=1 << 30,
                 partitions=None, cold_launches=100, mode="direct"):
    """Time paged decode over `case`: `steps` launches back to back between one
    event pair, each reading another copy of the KV pool (copies rotate, > 1
    GiB in all, so every step streams its KV from HBM), then `cold_launches`
    more, each between its own event pair after a 1 GiB cache-flushing write,
    for the per-launch distribution.  Every call passes the per-sequence
    status array (the full operator contract).  mode "balanced" passes the
    load-balanced mode's workspace."""
    kv = case.kv
    B, hq, _ = case.q.shape
    P = case.num_partitions if partitions is None else partitions
    pool_bytes = kv.k_pool.nbytes * 2
    ncopies = max(1, min(16, math.ceil(copies_bytes / max(pool_bytes, 1)) + 1))
    kps = [dev(kv.k_pool)]
    vps = [dev(kv.v_pool)]
    for _ in range(ncopies - 1):
        kps.append(kps[0].clone())
        vps.append(vps[0].clone())
    q = dev(case.q)
    o = torch.empty_like(q)
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    indptr, ids, lens = dev(kv.page_indptr), dev(kv.page_indices), dev(kv.seq_lens)
    if mode == "balanced":
        nbytes = oxa.oxa_paged_decode_balanced_workspace_bytes(B, hq, P)
        assert nbytes > 0
    else:
        nbytes = oxa.oxa_paged_decode_workspace_bytes(B, hq, P)
    ws = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device="cuda") if nbytes else None
    stream = torch.cuda.current_stream()

    def call(i):
        j = i % ncopies
        rc = oxa.oxa_paged_decode(q, kps[j], vps[j], indptr, ids, lens, o,
                                  max_seq_len=case.max_seq_len, sm_scale=case.sm_scale,
                                  layout=kv.layout, num_kv_heads=kv.num_kv_heads,
                                  num_partitions=P, workspace=ws, status=status)
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # throughput: `steps` launches back to back, one event pair around them all
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        call(i + warmup)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    assert (status == 0).all().item(), "decode status reports an invalid sequence"
    # distribution: cold launches, each between its own event pair (an event
    # record before and after a launch adds a few us to it)
    cold = cold_launch_samples(torch, stream, lambda i: call(i + warmup + steps),
                               max(cold_launches, steps), scratch)
    return dict(total_ms=total_ms, launch_ms=cold, bytes=decode_bytes(case), copies=ncopies,
                partitions=P, steps=steps)


def bench_prefill_ragged(torch, oxa, case, iters, warmup):
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    o = torch.empty_like(q)
    qi, ki = dev(case.qo_indptr), dev(case.kv_indptr)
    qlens = np.diff(case.qo_indptr)
    klens = np.diff(case.kv_indptr)
    stream = torch.cuda.current_stream()

    def call(i):
        rc = oxa.oxa_ragged_prefill(q, k, v, qi, ki, o, max_qo_len=int(qlens.max()),
                                    max_kv_len=int(klens.max()), sm_scale=case.sm_scale,
                                    causal=True)
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    for i in range(warmup):
        call(i)
    warm_clock(torch, lambda: call(0))
    timer = LaunchTimer(torch, stream, iters)
    timer.run(call, iters)
    ms = timer.launch_ms(iters)
    return dict(launch_ms=ms, flops=causal_flops(qlens, klens, case.num_qo_heads))


def bench_append_and_paged_prefill(torch, oxa, case, iters, warmup):
    kv = case.kv
    q_in = dev(case.q)
    q_rot = torch.empty_like(q_in)
    k_in, v_in = dev(case.k), dev(case.v)
    bi, pos = dev(case.batch_indices), dev(case.positions)
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    indptr, ids, rc_t = dev(kv.page_indptr), dev(kv.page_indices), dev(case.page_refcounts)
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    lens = dev(kv.seq_lens)
    qoi = dev(case.qo_indptr)
    o = torch.empty_like(q_in)
    stream = torch.cuda.current_stream()
    hkv = kv.num_kv_heads

    ws_a = torch.empty(oxa.oxa_paged_append_rope_workspace_bytes(case.k.shape[0]),
                       dtype=torch.uint8, device="cuda")

    def append(i):
        rc = oxa.oxa_paged_append_rope(q_in, q_rot, k_in, v_in, bi, pos, kp, vp, indptr, ids, rc_t,
                                       status, layout=kv.layout, rope_theta=case.rope_theta,
                                       workspace=ws_a)
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    max_len = int(kv.seq_lens.max())

    def prefill(i):
        rc = oxa.oxa_paged_prefill(q_rot, qoi, kp, vp, indptr, ids, lens, o, max_qo_len=max_len,
                                   max_seq_len=max_len, sm_scale=case.sm_scale, layout=kv.layout,
                                   num_kv_heads=hkv, causal=True)
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    for i in range(warmup):
        append(i)
        prefill(i)
    warm_clock(torch, lambda: prefill(0), seconds=0.2)
    warm_clock(torch, lambda: append(0), seconds=0.1)
    ta = LaunchTimer(torch, stream, iters)
    ta.run(append, iters)
    a_ms = ta.launch_ms(iters)
    warm_clock(torch, lambda: prefill(0), seconds=0.1)
    tp = LaunchTimer(torch, stream, iters)
    tp.run(prefill, iters)
    p_ms = tp.launch_ms(iters)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, -1]

    # the plain append of the same tokens into the same pages (timed last: it
    # leaves unrotated k in the pages)
    def plain(i):
        rc = oxa.oxa_paged_append(k_in, v_in, bi, pos, kp, vp, indptr, ids, rc_t, status,
                                  layout=kv.layout, workspace=ws_a)
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    for i in range(warmup):
        plain(i)
    warm_clock(torch, lambda: plain(0), seconds=0.1)
    tq = LaunchTimer(torch, stream, iters)
    tq.run(plain, iters)
    q_ms = tq.launch_ms(iters)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, -1]
    nnz, hq, d = case.q.shape
    kv_bytes = (nnz * hkv * d * 2 * 2 * 2           # k, v read + written into pages
                + nnz * 4 * 2                       # positions + batch indices
                + nnz // 16 * 4 * 2)                # page ids + refcounts, once per page
    append_bytes = nnz * hq * d * 2 * 2 + kv_bytes  # + q read and q_out written
    qlens = np.diff(case.qo_indptr)
    return dict(append_ms=a_ms, append_bytes=append_bytes, prefill_ms=p_ms,
                prefill_flops=causal_flops(qlens, kv.seq_lens, hq), plain_ms=q_ms,
                plain_bytes=kv_bytes)


def bench_pages_shapes(torch, oxa, W, iters=200, warmup=20):
    """Per-call latency of the four attention shapes that the Oxide Infer README's
    Performance snapshot prints (HIP events around each launch, inputs resident,
    so small working sets sit in cache, as in a serving loop).  Head counts are
    not printed there: 32 q heads, 32 kv heads for MHA and 8 for GQA4.

    A prefill shape is timed with the optional workspace (small calls may then
    split their keys) and without it ("_unsplit"), the two forms alternating
    call by call so that both see the same clock; the pair is timed twice, in
    both orders, and each form reports the median over both passes."""
    stream = torch.cuda.current_stream()
    res = {}

    def graph_us(call):
        # the same call captured once in a HIP graph and replayed
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            call(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(0)
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        tg = LaunchTimer(torch, stream, iters)
        tg.run(lambda i: g.replay(), iters)
        return round(float(np.median(tg.launch_ms(iters))) * 1e3, 2)

    def timed(forms):
        """forms: [(name, call)]; calls alternate within each pass."""
        for _, call in forms:
            for i in range(warmup):
                call(i)
        warm_clock(torch, lambda: [c(0) for _, c in forms], seconds=0.2)
        samples = {name: [] for name, _ in forms}
        for order in (forms, forms[::-1]):
            pairs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in order] for _ in range(iters)]
            for i in range(iters):
                for (name, call), (a, b) in zip(order, pairs[i]):
                    a.record(stream)
                    call(i)
                    b.record(stream)
            torch.cuda.synchronize()
            for i in range(iters):
                for (name, _), (a, b) in zip(order, pairs[i]):
                    samples[name].append(a.elapsed_time(b))
        for name, call in forms:
            ms = np.array(samples[name])
            res[name] = {"us_median": round(float(np.median(ms)) * 1e3, 2),
                         "us_p10_p90": [round(float(x) * 1e3, 2) for x in np.percentile(ms, [10, 90])],
                         "graph_us_median": graph_us(call)}

    def check(rc):
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    c = W.pages_decode_b1_kv1()
    kv = c.kv
    q = dev(c.q)
    o = torch.empty_like(q)
    args = (dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr), dev(kv.page_indices),
            dev(kv.seq_lens))
    timed([("decode_mha_b1_kv1", lambda i: check(oxa.oxa_paged_decode(
        q, *args, o, max_seq_len=1, sm_scale=c.sm_scale, layout=kv.layout,
        num_kv_heads=kv.num_kv_heads)))])

    # prefill calls pass the optional workspace, with which small calls split
    # their keys over more CUs; the "_unsplit" forms are the same calls without
    def workspace(nbytes):
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    for name, rc_ in (("ragged_mha_q16_kv16", W.pages_ragged_mha_q16()),
                      ("ragged_gqa4_q32+64_kv256+1024", W.pages_ragged_gqa4())):
        qr, kr, vr = dev(rc_.q), dev(rc_.k), dev(rc_.v)
        orr = torch.empty_like(qr)
        qi, ki = dev(rc_.qo_indptr), dev(rc_.kv_indptr)
        mq, mk = int(np.diff(rc_.qo_indptr).max()), int(np.diff(rc_.kv_indptr).max())
        ws = workspace(oxa.oxa_ragged_prefill_workspace_bytes(len(rc_.qo_indptr) - 1,
                                                              qr.shape[0], qr.shape[1]))
        timed([(name + suffix,
                lambda i, qr=qr, kr=kr, vr=vr, orr=orr, qi=qi, ki=ki, mq=mq, mk=mk, c=rc_, w=w:
                check(oxa.oxa_ragged_prefill(qr, kr, vr, qi, ki, orr, max_qo_len=mq,
                                             max_kv_len=mk, sm_scale=c.sm_scale, causal=True,
                                             workspace=w)))
               for suffix, w in (("", ws), ("_unsplit", None))])

    pc = W.pages_paged_gqa4()
    kv = pc.kv
    qp = dev(pc.q)
    op = torch.empty_like(qp)
    pargs = (dev(pc.qo_indptr), dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr),
             dev(kv.page_indices), dev(kv.seq_lens))
    ws = workspace(oxa.oxa_paged_prefill_workspace_bytes(2, qp.shape[0], qp.shape[1]))
    timed([("paged_gqa4_q32+64_kv256+1024" + suffix, lambda i, w=w: check(oxa.oxa_paged_prefill(
        qp, *pargs, op, max_qo_len=64, max_seq_len=1024, sm_scale=pc.sm_scale,
        layout=kv.layout, num_kv_heads=kv.num_kv_heads, causal=True, workspace=w)))
           for suffix, w in (("", ws), ("_unsplit", None))])
    return res


def bench_merge(torch, oxa, iters=30, warmup=5):
    """Attention-state merges at serving sizes, inputs cold (two copies rotate):
    a cascade pair over 16384 rows x 32 heads (bf16 states, the prefill-batch
    shape), and 8 f32 partial states over 512 rows x 32 heads into bf16."""
    stream = torch.cuda.current_stream()
    res = {}

    def run(name, make, call, nbytes):
        bufs = [make(i) for i in range(2)]
        for i in range(warmup):
            call(bufs[i % 2])
        warm_clock(torch, lambda: call(bufs[0]), seconds=0.1)
        t = LaunchTimer(torch, stream, iters)
        t.run(lambda i: call(bufs[i % 2]), iters)
        ms = float(np.mean(t.launch_ms(iters)))
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes}

    def check(rc):
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    R, H = 16384, 32
    def make_pair(i):
        g = torch.Generator(device="cuda").manual_seed(3000 + i)
        va = torch.randn(R, H, 128, device="cuda", generator=g).to(torch.bfloat16)
        vb = torch.randn(R, H, 128, device="cuda", generator=g).to(torch.bfloat16)
        la = torch.randn(R, H, device="cuda", generator=g) * 4
        lb = torch.randn(R, H, device="cuda", generator=g) * 4
        return va, la, vb, lb, torch.empty_like(va), torch.empty_like(la)
    run("merge_pair_bf16_r16384_h32", make_pair,
        lambda b: check(oxa.oxa_merge_state_pair(*b)), R * H * (3 * 256 + 3 * 4))

    R2, S2 = 512, 8
    def make_multi(i):
        g = torch.Generator(device="cuda").manual_seed(3100 + i)
        v = torch.randn(R2, S2, H, 128, device="cuda", generator=g)
        lse = torch.randn(R2, S2, H, device="cuda", generator=g) * 4
        return v, lse, torch.empty(R2, H, 128, dtype=torch.bfloat16, device="cuda"), \
            torch.empty(R2, H, device="cuda")
    run("merge_f32x8_to_bf16_r512_h32", make_multi,
        lambda b: check(oxa.oxa_merge_states(*b)), R2 * H * (S2 * (512 + 4) + 256 + 4))
    return res


def bench_rope(torch, oxa, iters=20, warmup=3):
    """Standalone NeoX RoPE of q and k at the long-prefill shape: 32768 tokens,
    32 q / 8 kv heads, positions 0..16383 twice (out of place)."""
    nnz, hq, hkv = 32768, 32, 8
    q = torch.randn(nnz, hq, 128, device="cuda").to(torch.bfloat16)
    k = torch.randn(nnz, hkv, 128, device="cuda").to(torch.bfloat16)
    pos = dev(np.tile(np.arange(16384, dtype=np.int32), 2))
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    stream = torch.cuda.current_stream()

    def call(i):
        rc = oxa.oxa_rope_neox(q, qo, k, ko, pos, rope_theta=10000.0)
        if rc != 0:
            raise RuntimeError(oxa.status_string(rc))

    for i in range(warmup):
        call(i)
    warm_clock(torch, lambda: call(0), seconds=0.1)
    t = LaunchTimer(torch, stream, iters)
    t.run(call, iters)
    ms = float(np.mean(t.launch_ms(iters)))
    nbytes = nnz * (hq + hkv) * 256 * 2 + nnz * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"rope_neox_32768_tok_32q_8kv": {"us": round(ms * 1e3, 1), "GB/s": round(gbs, 1),
                                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                            "bytes": nbytes}}


def host_info():
    """Host cores, the BLAS pool's threads and the CPU model string."""
    from threadpoolctl import threadpool_info
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "blas_threads": max(blas) if blas else 1,
            "cpu_model": model}


def cpu_baseline(cases):
    """The oracle (float64 numpy, as it stands) timed on this host's cores, its
    BLAS pool at its default size, on each workload or a stated sample of it:
    paged decode (batch-1 MHA, batch-32 GQA4, long MQA) median of 5 whole
    runs; ragged GQA4 prefill, RoPE + append and the long paged prefill once
    each on a sample (rates scaled by the sample's share of the work)."""
    from oracle import attention as A
    from oracle import rope as R
    import workloads as W
    info = host_info()
    out = {}

    def med5(fn):
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    for name, key in (("decode_mha_b1_l256", "c1"), ("decode_gqa4_b32", "c2"),
                      ("decode_mqa_b8_l32768", "c3")):
        case = cases[key]
        kv = case.kv
        t = med5(lambda: A.paged_decode(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                        kv.page_indices, kv.seq_lens, case.sm_scale))
        out[name] = {"s": round(t, 4), "GB/s": round(decode_bytes(case) / t / 1e9, 3),
                     "sample": "whole workload, median of 5"}
    rng = np.random.default_rng(7)
    c4 = cases["c4"]
    rows = np.sort(rng.choice(len(c4.q), 256, replace=False))
    qlens, klens = np.diff(c4.qo_indptr), np.diff(c4.kv_indptr)
    t0 = time.perf_counter()
    A.ragged_prefill(c4.q, c4.k, c4.v, c4.qo_indptr, c4.kv_indptr, c4.sm_scale, True, rows=rows)
    t = time.perf_counter() - t0
    fl = sampled_causal_flops(rows, c4.qo_indptr, klens, c4.num_qo_heads)
    out["prefill_ragged_gqa4_4seq"] = {"s": round(t, 3), "GFLOP/s": round(fl / t / 1e9, 3),
                                       "sample": "256 random query rows of 7680 (all heads)"}
    c5 = cases["c5"]
    small = W.append_case(1005, seq_lens=[1024, 1024], num_qo_heads=32, num_kv_heads=8)
    kv = small.kv
    t0 = time.perf_counter()
    R.paged_append_rope(small.q, small.k, small.v, small.batch_indices, small.positions,
                        kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr, kv.page_indices,
                        small.page_refcounts, small.rope_theta)
    t = time.perf_counter() - t0
    nbytes = 2048 * (32 * 256 * 2 + 8 * 256 * 4 + 8) + 128 * 8
    out["rope_append_2x16384"] = {"s": round(t, 3), "GB/s": round(nbytes / t / 1e9, 4),
                                  "sample": "2 x 1024 tokens of the same shape (32 q / 8 kv "
                                            "heads, exclusive pages)"}
    kv = c5.kv
    rows = np.sort(rng.choice(len(c5.q), 64, replace=False))
    t0 = time.perf_counter()
    A.paged_prefill(c5.q, c5.qo_indptr, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                    kv.page_indices, kv.seq_lens, c5.sm_scale, True, rows=rows)
    t = time.perf_counter() - t0
    fl = sampled_causal_flops(rows, c5.qo_indptr, kv.seq_lens, 32)
    out["prefill_paged_gqa4_2x16384"] = {"s": round(t, 3), "GFLOP/s": round(fl / t / 1e9, 3),
                                         "sample": "64 random query rows of 32768 (all heads)"}
    c2 = out["decode_gqa4_b32"]
    return dict(value=c2["GB/s"], unit="GB/s", cores=info["blas_threads"], kind="oracle",
                sample="whole batch-32 GQA4 decode workload, median of 5 runs (numpy float64, "
                       "BLAS pool at its default size; the other workloads under 'configs')",
                host=info, configs=out)


def sampled_causal_flops(rows, qo_indptr, kv_lens, hq, d=128):
    """Matrix flops of the given packed query rows (bottom-right causal)."""
    qo_indptr = np.asarray(qo_indptr)
    total = 0
    for r in rows:
        b = int(np.searchsorted(qo_indptr, r, side="right")) - 1
        qlen = int(qo_indptr[b + 1] - qo_indptr[b])
        i = int(r - qo_indptr[b])
        total += i + 1 + int(kv_lens[b]) - qlen
    return 4 * d * hq * total


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=ROWS, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-partitions", type=int, default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library's hot path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_attention_02_amd as oxa
    import workloads as W
    if not os.path.exists(oxa.LIB_PATH):
        from paged_attention_02_amd import build as _b
        _b.build()
    oxa.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    only = args.only
    out = {}

    decode_P = args.decode_partitions
    if decode_P is None:
        decode_P = int(os.environ.get("OXA_BENCH_DECODE_P", "1"))
    cases = {"c2": W.decode_gqa4_batch(num_partitions=decode_P)}
    case2 = cases["c2"]
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")  # cache-flushing writes
    if only in (None, "decode"):
        log("decode: batch-32 GQA4")
        out["decode"] = bench_decode(torch, oxa, W, case2, args.steps, args.warmup, scratch)
        log("decode: batch-32 GQA4, load-balanced mode")
        out["decode_balanced"] = bench_decode(torch, oxa, W, case2, args.steps, args.warmup,
                                              scratch, mode="balanced")
    if only in (None, "decode_mha"):
        log("decode_mha: batch-1 MHA, 256 tokens")
        cases["c1"] = W.decode_mha_small()
        out["decode_mha"] = bench_decode(torch, oxa, W, cases["c1"], 100, 10, scratch)
    if only in (None, "decode_mqa"):
        log("decode_mqa: batch-8 MQA, 32768 tokens, 16 partitions")
        cases["c3"] = W.decode_mqa_long()
        out["decode_mqa"] = bench_decode(torch, oxa, W, cases["c3"], 30, 5, scratch)
        log("decode_mqa: load-balanced mode")
        out["decode_mqa_balanced"] = bench_decode(torch, oxa, W, cases["c3"], 30, 5, scratch,
                                                  mode="balanced")
    if only in (None, "decode_skewed"):
        log("decode_skewed: batch-32 GQA4, one 32768-token sequence and 31 of 1024, both modes")
        sk = W.decode_skewed()
        out["decode_skewed"] = bench_decode(torch, oxa, W, sk, 30, 5, scratch, cold_launches=30)
        out["decode_skewed_balanced"] = bench_decode(torch, oxa, W, sk, 30, 5, scratch,
                                                     cold_launches=30, mode="balanced")
    if only in (None, "prefill_ragged"):
        log("prefill_ragged: GQA4 {512,1024,2048,4096}")
        cases["c4"] = W.ragged_gqa4_prefill()
        out["prefill_ragged"] = bench_prefill_ragged(torch, oxa, cases["c4"], 20, 3)
    if only in (None, "append", "prefill_paged"):
        log("append + paged prefill: 2 x 16384 tokens")
        cases["c5"] = W.rope_append_prefill()
        out["long"] = bench_append_and_paged_prefill(torch, oxa, cases["c5"], 10, 2)
    del scratch

    if only in (None, "pages_shapes"):
        log("pages_shapes: the four printed attention shapes, per-call latency")
        out["pages_shapes"] = bench_pages_shapes(torch, oxa, W)

    if only in (None, "merge"):
        log("merge: attention-state merges (cascade pair, 8 f32 partials)")
        out["merge"] = bench_merge(torch, oxa)

    if only in (None, "rope"):
        log("rope: standalone NeoX RoPE, 32768 tokens")
        out["rope"] = bench_rope(torch, oxa)

    if only == "copy":
        # a plain device copy of known size: the reference for scaling the HBM
        # byte counters (FETCH_SIZE / WRITE_SIZE) read under rocprofv3
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {n} bytes")

    line = {
        "metric": "paged-decode HBM GB/s (% peak) + causal-prefill TFLOPS (% bf16 MFMA peak)",
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    if "decode" in out:
        r = out["decode"]
        step_ms = r["total_ms"] / args.steps    # mean launch duration, back to back
        achieved = r["bytes"] / (step_ms * 1e-3) / 1e9
        traffic = profiled_traffic("decode.hip", "paged_decode_gqa4_batch32.md")
        line.update({
            "value": round(r["bytes"] / (step_ms * 1e-3) / 1e9, 1),
            "ms_per_step": round(step_ms, 5),
            "config": {"workload": "paged batch decode GQA4: batch 32, 32 q / 8 kv heads, "
                                   "head_dim 128, page 16, seq_lens U[512,4096] (seed 1002), "
                                   "shuffled NHD pool, bf16 N(0,1)",
                       "seq_tokens": int(case2.kv.seq_lens.sum()),
                       "num_partitions": r["partitions"],
                       "pool_copies_rotated": r["copies"],
                       "algorithmic_bytes_per_step": r["bytes"]},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic,
                         "kernel": "paged_decode_kernel" + ("" if r["partitions"] == 1 else
                                                            " + merge_states_kernel"),
                         "us_per_launch": round(step_ms * 1e3, 2),
                         "cold_launch_event_pairs_us_p10_p50_p90":
                             [round(float(x) * 1e3, 2) for x in
                              np.percentile(r["launch_ms"], [10, 50, 90])]},
        })
    rows = {}

    def cold_stats(r):
        ms = np.asarray(r["launch_ms"])
        return {"cold_us_p10_p50_p90": [round(float(x) * 1e3, 2)
                                        for x in np.percentile(ms, [10, 50, 90])],
                "cold_us_samples": [round(float(x) * 1e3, 2) for x in ms]}

    if "decode" in out:
        rows["decode_gqa4_b32_cold_launches"] = cold_stats(out["decode"])
    if "decode_mha" in out:
        r = out["decode_mha"]
        lm = r["total_ms"] / r["steps"]
        rows["decode_mha_b1_l256"] = {"us": round(lm * 1e3, 2),
                                      "GB/s": round(r["bytes"] / (lm * 1e-3) / 1e9, 1),
                                      **cold_stats(r)}
    def decode_row(r):
        lm = r["total_ms"] / r["steps"]
        gbs = r["bytes"] / (lm * 1e-3) / 1e9
        return {"us": round(lm * 1e3, 2), "GB/s": round(gbs, 1),
                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": r["bytes"], **cold_stats(r)}

    if "decode_balanced" in out:
        rows["decode_gqa4_b32_balanced_mode"] = decode_row(out["decode_balanced"])
    if "decode_mqa" in out:
        rows["decode_mqa_splitk_b8_l32768_p16"] = decode_row(out["decode_mqa"])
        rows["decode_mqa_splitk_b8_l32768_p16_balanced_mode"] = decode_row(
            out["decode_mqa_balanced"])
    if "decode_skewed" in out:
        rows["decode_skewed_gqa4_b32_direct_mode"] = decode_row(out["decode_skewed"])
        rows["decode_skewed_gqa4_b32_balanced_mode"] = decode_row(out["decode_skewed_balanced"])
    if "prefill_ragged" in out:
        r = out["prefill_ragged"]
        lm = float(np.mean(r["launch_ms"]))
        tf = r["flops"] / (lm * 1e-3) / 1e12
        rows["prefill_ragged_gqa4_4seq"] = {"us": round(lm * 1e3, 1), "TFLOPS": round(tf, 1),
                                            "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                            "flops": r["flops"]}
    if "long" in out:
        r = out["long"]
        am = float(np.mean(r["append_ms"]))
        pm = float(np.mean(r["prefill_ms"]))
        gbs = r["append_bytes"] / (am * 1e-3) / 1e9
        tf = r["prefill_flops"] / (pm * 1e-3) / 1e12
        rows["rope_append_2x16384"] = {"us": round(am * 1e3, 1), "GB/s": round(gbs, 1),
                                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                       "bytes": r["append_bytes"]}
        qm = float(np.mean(r["plain_ms"]))
        gq = r["plain_bytes"] / (qm * 1e-3) / 1e9
        rows["plain_append_2x16384"] = {"us": round(qm * 1e3, 1), "GB/s": round(gq, 1),
                                        "frac_hbm": round(gq / HBM_PEAK_GBS, 4),
                                        "bytes": r["plain_bytes"]}
        rows["prefill_paged_gqa4_2x16384"] = {"us": round(pm * 1e3, 1), "TFLOPS": round(tf, 1),
                                              "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                              "flops": r["prefill_flops"]}
        traffic = profiled_traffic("prefill.hip", "prefill_paged_gqa4_2x16384.md")
        line["prefill"] = {"metric": "causal-prefill TFLOPS", "value": round(tf, 1),
                           "unit": "TFLOP/s",
                           "workload": "paged causal prefill GQA4, 2 x 16384 tokens, 32 q / 8 kv "
                                       "heads, pages filled by the fused RoPE + append",
                           "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                        "traffic": traffic, "kernel": "prefill_kernel"}}
    if "pages_shapes" in out:
        rows["pages_shapes_latency"] = out["pages_shapes"]
    if "merge" in out:
        rows.update(out["merge"])
    if "rope" in out:
        rows.update(out["rope"])
    line["rows"] = rows
    if "value" not in line:
        line.update({"value": None, "ms_per_step": None, "config": {"workload": only}})
    if only is None and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cases)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
