"""HIP graph capture and replay of every entry point.

The calls only enqueue kernels on the caller's stream (no allocation, no
synchronisation, no memset), so a captured call replays with fixed addresses.
Each test captures a call once, then replays it several times.  Between
replays it changes the graph's inputs in place and runs the same call eagerly
on other outputs, with synchronisations; every replay must equal the eager
result bit for bit.  Invalid page ids and a shared page, planted between
replays, must be flagged in the status array by the replay itself.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_helpers import assert_attention_close, dev, host, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu

REPLAYS = 3


def capture(fn):
    """Warm fn up eagerly on a side stream, then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def ok(rc):
    assert rc == oxa.OXA_OK, oxa.status_string(rc)


@pytest.mark.parametrize("P", [1, 3])
def test_decode_graph_replays_equal_eager(P):
    case = W.decode_gqa4_batch(num_partitions=P)
    kv = case.kv
    ensure_built()
    B, hq, _ = case.q.shape
    q = dev(case.q)
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    indptr, ids, lens = dev(kv.page_indptr), dev(kv.page_indices), dev(kv.seq_lens)
    nbytes = oxa.oxa_paged_decode_workspace_bytes(B, hq, P)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda") if nbytes else None
    outs = {k: (torch.empty_like(q), torch.empty(B, hq, dtype=torch.float32, device="cuda"),
                torch.full((B,), -1, dtype=torch.int32, device="cuda")) for k in ("g", "e")}

    def call(which):
        o, lse, st = outs[which]
        ok(oxa.oxa_paged_decode(q, kp, vp, indptr, ids, lens, o, max_seq_len=case.max_seq_len,
                                sm_scale=case.sm_scale, num_kv_heads=kv.num_kv_heads,
                                num_partitions=P, workspace=ws, lse=lse, status=st))

    note(f"graph decode P={P}: capture")
    g = capture(lambda: call("g"))
    rng = np.random.default_rng(2500 + P)
    cur_lens = kv.seq_lens.copy()
    for rep in range(REPLAYS):
        new_q = W.bf16_normal(rng, case.q.shape)
        cur_lens = np.maximum(1, cur_lens - rng.integers(0, 300, B)).astype(np.int32)
        q.copy_(dev(new_q))
        lens.copy_(dev(cur_lens))
        note(f"graph decode P={P}: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        for a, b in zip(outs["g"], outs["e"]):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        assert (host(outs["g"][2]) == 0).all()
    o_ref, lse_ref = A.paged_decode(new_q, kv.k_pool, kv.v_pool, "NHD", kv.page_indptr,
                                    kv.page_indices, cur_lens, case.sm_scale)
    assert_attention_close(host_bits(outs["g"][0]), o_ref, f"graph decode P={P}")

    # a page id out of range, planted between replays, is caught by the replay
    bad_b = 5
    slot = int(kv.page_indptr[bad_b])
    ids[slot] = kv.num_pages + 11
    note(f"graph decode P={P}: replay with a bad page id")
    g.replay()
    torch.cuda.synchronize()
    st = host(outs["g"][2])
    assert st[bad_b] == oxa.OXA_DEV_PAGE_RANGE
    assert (np.delete(st, bad_b) == 0).all()
    ids[slot] = int(kv.page_indices[slot])
    g.replay()
    call("e")
    torch.cuda.synchronize()
    assert (host(outs["g"][2]) == 0).all()
    assert torch.equal(outs["g"][0], outs["e"][0])


def test_ragged_prefill_graph_replays_equal_eager():
    case = W.ragged_gqa4_prefill()
    ensure_built()
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    qi, ki = dev(case.qo_indptr), dev(case.kv_indptr)
    B = len(case.qo_indptr) - 1
    outs = {w: (torch.empty_like(q), torch.empty(q.shape[0], q.shape[1], dtype=torch.float32,
                                                 device="cuda"),
                torch.full((B,), -1, dtype=torch.int32, device="cuda")) for w in ("g", "e")}

    def call(which):
        o, lse, st = outs[which]
        ok(oxa.oxa_ragged_prefill(q, k, v, qi, ki, o, max_qo_len=4096, max_kv_len=4096,
                                  sm_scale=case.sm_scale, causal=True, lse=lse, status=st))

    note("graph ragged prefill: capture")
    g = capture(lambda: call("g"))
    rng = np.random.default_rng(2600)
    for rep in range(REPLAYS):
        q.copy_(dev(W.bf16_normal(rng, case.q.shape)))
        v.copy_(dev(W.bf16_normal(rng, case.v.shape)))
        note(f"graph ragged prefill: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        for a, b in zip(outs["g"], outs["e"]):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        assert (host(outs["g"][2]) == 0).all()


def test_long_paged_prefill_graph_replays_and_rejects_invalid_pages():
    """Paged causal GQA4 prefill over 2 x 16384 tokens, captured once."""
    case = W.rope_append_prefill()
    kv = case.kv
    ensure_built()
    q = dev(case.q)
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    qoi, indptr, ids, lens = (dev(case.qo_indptr), dev(kv.page_indptr), dev(kv.page_indices),
                              dev(kv.seq_lens))
    outs = {w: (torch.empty_like(q), torch.full((2,), -1, dtype=torch.int32, device="cuda"))
            for w in ("g", "e")}

    def call(which):
        o, st = outs[which]
        ok(oxa.oxa_paged_prefill(q, qoi, kp, vp, indptr, ids, lens, o, max_qo_len=16384,
                                 max_seq_len=16384, sm_scale=case.sm_scale, layout=kv.layout,
                                 num_kv_heads=kv.num_kv_heads, causal=True, status=st))

    note("graph paged prefill 2x16384: capture")
    g = capture(lambda: call("g"))
    rng = np.random.default_rng(2700)
    for rep in range(REPLAYS):
        rows = rng.integers(0, q.shape[0], 64)
        q[torch.from_numpy(rows).cuda()] = dev(W.bf16_normal(rng, (64,) + tuple(q.shape[1:])))
        note(f"graph paged prefill: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        assert torch.equal(outs["g"][0], outs["e"][0]), f"replay {rep} differs from eager"
        assert host(outs["g"][1]).tolist() == [0, 0]
    # invalid page id in sequence 1, planted between replays
    slot = int(kv.page_indptr[1]) + 321
    ids[slot] = -3
    note("graph paged prefill: replay with a negative page id")
    g.replay()
    torch.cuda.synchronize()
    assert host(outs["g"][1]).tolist() == [0, oxa.OXA_DEV_PAGE_RANGE]
    ids[slot] = int(kv.page_indices[slot])
    g.replay()
    call("e")
    torch.cuda.synchronize()
    assert host(outs["g"][1]).tolist() == [0, 0]
    assert torch.equal(outs["g"][0], outs["e"][0])


@pytest.mark.parametrize("plain", [False, True])
def test_append_graph_replays_equal_eager_and_reject_a_shared_page(plain):
    case = W.append_case(2800, seq_lens=[300, 37, 129], num_qo_heads=32, num_kv_heads=8,
                         extra_pages=1, spare_pages=3)
    kv = case.kv
    ensure_built()
    nnz = case.k.shape[0]
    q_in, k_in, v_in = dev(case.q), dev(case.k), dev(case.v)
    bi, pos = dev(case.batch_indices), dev(case.positions)
    indptr, ids, refc = dev(kv.page_indptr), dev(kv.page_indices), dev(case.page_refcounts)
    ws = torch.empty(oxa.oxa_paged_append_rope_workspace_bytes(nnz), dtype=torch.uint8,
                     device="cuda")
    state = {w: dict(kp=dev(kv.k_pool), vp=dev(kv.v_pool), q=torch.empty_like(q_in),
                     st=torch.full((2,), 7, dtype=torch.int32, device="cuda"))
             for w in ("g", "e")}

    def call(which):
        t = state[which]
        if plain:   # the plain append (no RoPE, no q)
            ok(oxa.oxa_paged_append(k_in, v_in, bi, pos, t["kp"], t["vp"], indptr, ids, refc,
                                    t["st"], layout=kv.layout, workspace=ws))
        else:
            ok(oxa.oxa_paged_append_rope(q_in, t["q"], k_in, v_in, bi, pos, t["kp"], t["vp"],
                                         indptr, ids, refc, t["st"], layout=kv.layout,
                                         rope_theta=case.rope_theta, workspace=ws))

    note(f"graph append plain={plain}: capture")
    g = capture(lambda: call("g"))
    rng = np.random.default_rng(2900)
    for rep in range(REPLAYS):
        k_in.copy_(dev(W.bf16_normal(rng, case.k.shape)))
        v_in.copy_(dev(W.bf16_normal(rng, case.v.shape)))
        note(f"graph append: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        for key in ("kp", "vp", "st") + (() if plain else ("q",)):
            assert torch.equal(state["g"][key], state["e"][key]), f"replay {rep}: {key}"
        assert host(state["g"]["st"]).tolist() == [0, -1]
    # a target page that another sequence shares (refcount 2): the replay
    # writes nothing and names the first token that targets it
    page = int(kv.page_indices[kv.page_indptr[1]])
    before_k = state["g"]["kp"].clone()
    before_v = state["g"]["vp"].clone()
    k_in.copy_(dev(W.bf16_normal(rng, case.k.shape)))
    refc[page] = 2
    note("graph append: replay with a shared page")
    g.replay()
    torch.cuda.synchronize()
    assert host(state["g"]["st"]).tolist() == [oxa.OXA_DEV_NOT_EXCLUSIVE, 300]
    assert torch.equal(state["g"]["kp"], before_k) and torch.equal(state["g"]["vp"], before_v)
    refc[page] = 1
    g.replay()
    call("e")
    torch.cuda.synchronize()
    assert host(state["g"]["st"]).tolist() == [0, -1]
    assert torch.equal(state["g"]["kp"], state["e"]["kp"])


def test_merge_graph_replays_equal_eager():
    R, S, H = 300, 6, 16
    case = W.merge_case(3000, R, S, H, dtype="f32")
    ensure_built()
    v, lse = dev(case.v), dev(case.lse)
    va, la = dev(case.v[:, 0]), dev(case.lse[:, 0])
    vb, lb = dev(case.v[:, 1]), dev(case.lse[:, 1])
    outs = {w: (torch.empty(R, H, 128, dtype=torch.bfloat16, device="cuda"),
                torch.empty(R, H, dtype=torch.float32, device="cuda"),
                torch.empty(R, H, 128, dtype=torch.float32, device="cuda"),
                torch.empty(R, H, dtype=torch.float32, device="cuda")) for w in ("g", "e")}

    def call(which):
        o, lo, o2, lo2 = outs[which]
        ok(oxa.oxa_merge_states(v, lse, o, lo))
        ok(oxa.oxa_merge_state_pair(va, la, vb, lb, o2, lo2))

    note("graph merge: capture")
    g = capture(lambda: call("g"))
    rng = np.random.default_rng(3001)
    for rep in range(REPLAYS):
        # new live lse values; empty states (NaN v) stay empty
        new_lse = (rng.standard_normal(case.lse.shape) * 4).astype(np.float32)
        new_lse[np.isneginf(case.lse)] = -np.inf
        lse.copy_(dev(new_lse))
        new_va = rng.standard_normal(va.shape).astype(np.float32)
        va.copy_(dev(new_va))
        note(f"graph merge: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        for a, b in zip(outs["g"], outs["e"]):
            assert torch.equal(a, b), f"replay {rep} differs from eager"


def test_rope_graph_replays_equal_eager():
    rng = np.random.default_rng(3100)
    nnz, hq, hkv = 4096, 32, 8
    q = dev(W.bf16_normal(rng, (nnz, hq, 128)))
    k = dev(W.bf16_normal(rng, (nnz, hkv, 128)))
    pos = dev(rng.integers(0, 32768, nnz).astype(np.int32))
    outs = {w: (torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)) for w in ("g", "e")}
    ensure_built()

    def call(which):
        qo, ko, ko2 = outs[which]
        ok(oxa.oxa_rope_neox(q, qo, k, ko, pos))
        ok(oxa.oxa_rope_llama31(None, None, k, ko2, pos))

    note("graph rope: capture")
    g = capture(lambda: call("g"))
    for rep in range(REPLAYS):
        pos.copy_(dev(rng.integers(-70000, 70000, nnz).astype(np.int32)))
        k.copy_(dev(W.bf16_normal(rng, (nnz, hkv, 128))))
        note(f"graph rope: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        for a, b in zip(outs["g"], outs["e"]):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
