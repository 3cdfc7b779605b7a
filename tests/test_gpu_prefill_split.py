"""Small prefill calls with a workspace: their keys are cut into chunks that
run on more compute units, and the chunk states are merged.

Against the FP64 oracle: the printed GQA4 shapes (ragged, and paged in both
layouts with poisoned unused slots), non-causal attention, sequences too short
to reach every chunk (empty chunk states), one invalid sequence among valid
ones, a reused workspace (a second, smaller call after a first), and graph
replays against eager calls.  The workspace starts filled with NaN bytes; a
call that split must have overwritten some of them, and no NaN may reach o.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_helpers import assert_attention_close, assert_lse_close, dev, host, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu


def nan_workspace(nbytes):
    assert nbytes > 0, "the call is expected to be small enough to split"
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")


def assert_split_ran(ws):
    assert (ws != 0xFF).any(), "the workspace was not written: the call did not split"


def ragged(case, causal=True, max_kv_len=None, workspace="auto", status=True):
    ensure_built()
    q = dev(case.q)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    B = len(case.qo_indptr) - 1
    st = torch.full((B,), -1, dtype=torch.int32, device="cuda") if status else None
    if workspace == "auto":
        workspace = nan_workspace(
            oxa.oxa_ragged_prefill_workspace_bytes(B, q.shape[0], q.shape[1]))
    rc = oxa.oxa_ragged_prefill(q, dev(case.k), dev(case.v), dev(case.qo_indptr),
                                dev(case.kv_indptr), o,
                                max_qo_len=max(1, int(np.diff(case.qo_indptr).max())),
                                max_kv_len=max_kv_len or max(1, int(np.diff(case.kv_indptr).max())),
                                sm_scale=case.sm_scale, causal=causal, lse=lse, status=st,
                                workspace=workspace)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    return o, lse, st, workspace


def check_ragged(case, o, lse, causal=True, rows=None):
    o_ref, lse_ref = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                                      case.sm_scale, causal)
    got_o, got_l = host_bits(o), host(lse)
    if rows is not None:
        got_o, got_l, o_ref, lse_ref = got_o[rows], got_l[rows], o_ref[rows], lse_ref[rows]
    assert_attention_close(got_o, o_ref, "split prefill")
    assert_lse_close(got_l, lse_ref)


def test_split_ragged_printed_gqa4():
    case = W.pages_ragged_gqa4()
    note("split ragged prefill gqa4 32+64 over 256+1024")
    o, lse, st, ws = ragged(case)
    assert_split_ran(ws)
    assert (host(st) == 0).all()
    check_ragged(case, o, lse)
    # the unsplit call agrees within the same tolerance
    o1, lse1, _, _ = ragged(case, workspace=None)
    check_ragged(case, o1, lse1)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_split_paged_printed_gqa4(layout):
    case = W.pages_paged_gqa4(layout=layout, poison=True)
    ensure_built()
    kv = case.kv
    q = dev(case.q)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    status = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    ws = nan_workspace(oxa.oxa_paged_prefill_workspace_bytes(2, q.shape[0], q.shape[1]))
    note(f"split paged prefill gqa4 {layout}")
    rc = oxa.oxa_paged_prefill(q, dev(case.qo_indptr), dev(kv.k_pool), dev(kv.v_pool),
                               dev(kv.page_indptr), dev(kv.page_indices), dev(kv.seq_lens), o,
                               max_qo_len=64, max_seq_len=1024, sm_scale=case.sm_scale,
                               layout=layout, num_kv_heads=kv.num_kv_heads, causal=True, lse=lse,
                               status=status, workspace=ws)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert_split_ran(ws)
    assert host(status).tolist() == [0, 0]
    o_ref, lse_ref = A.paged_prefill(case.q, case.qo_indptr, kv.k_pool, kv.v_pool, layout,
                                     kv.page_indptr, kv.page_indices, kv.seq_lens,
                                     case.sm_scale, True)
    assert_attention_close(host_bits(o), o_ref, f"split paged gqa4 {layout}")
    assert_lse_close(host(lse), lse_ref)


def test_split_non_causal():
    case = W.ragged_case(4600, qo_lens=[7, 40, 1], kv_lens=[300, 500, 1000], num_qo_heads=16,
                         num_kv_heads=4)
    note("split ragged prefill non-causal")
    o, lse, st, ws = ragged(case, causal=False)
    assert_split_ran(ws)
    check_ragged(case, o, lse, causal=False)


def test_split_with_short_and_empty_sequences():
    """Sequences of 1 to 63 keys have one key tile: every chunk but one is
    empty (lse -inf), and the merge must drop them; empty sequences between."""
    qo = [1, 0, 3, 17, 0, 64, 2]
    kv = [1, 4, 3, 63, 0, 1000, 65]
    case = W.ragged_case(4601, qo_lens=qo, kv_lens=kv, num_qo_heads=8, num_kv_heads=2)
    note("split ragged prefill short and empty sequences")
    o, lse, st, ws = ragged(case)
    assert_split_ran(ws)
    assert (host(st) == 0).all()
    check_ragged(case, o, lse)


def test_split_with_an_invalid_sequence():
    """Sequence 1 has more keys than max_kv_len: its status says so and the
    other sequences' rows are still right (its own rows are unspecified)."""
    qo = [20, 30, 10]
    kv = [500, 900, 40]
    case = W.ragged_case(4602, qo_lens=qo, kv_lens=kv, num_qo_heads=32, num_kv_heads=8)
    note("split ragged prefill with an invalid sequence")
    o, lse, st, ws = ragged(case, max_kv_len=800)
    assert_split_ran(ws)
    assert host(st).tolist() == [0, oxa.OXA_DEV_SEQ_LEN, 0]
    rows = np.r_[0:20, 50:60]
    check_ragged(case, o, lse, rows=rows)


def test_split_workspace_reused_by_a_smaller_call():
    big = W.ragged_case(4603, qo_lens=[64, 64], kv_lens=[2000, 700], num_qo_heads=32,
                       num_kv_heads=8)
    small = W.ragged_case(4604, qo_lens=[5, 9], kv_lens=[130, 9], num_qo_heads=32,
                         num_kv_heads=8)
    ws = nan_workspace(oxa.oxa_ragged_prefill_workspace_bytes(2, 128, 32))
    assert oxa.oxa_ragged_prefill_workspace_bytes(2, 14, 32) <= ws.numel()
    note("split ragged prefill: workspace reuse, first call")
    o, lse, _, _ = ragged(big, workspace=ws)
    assert_split_ran(ws)
    check_ragged(big, o, lse)
    note("split ragged prefill: workspace reuse, second smaller call")
    o, lse, _, _ = ragged(small, workspace=ws)
    check_ragged(small, o, lse)


def test_split_graph_replays_equal_eager():
    case = W.pages_ragged_gqa4()
    ensure_built()
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    qi, ki = dev(case.qo_indptr), dev(case.kv_indptr)
    nb = oxa.oxa_ragged_prefill_workspace_bytes(2, q.shape[0], q.shape[1])
    outs = {w: (torch.empty_like(q), torch.empty(q.shape[0], q.shape[1], dtype=torch.float32,
                                                 device="cuda"), nan_workspace(nb))
            for w in ("g", "e")}

    def call(which):
        o, lse, ws = outs[which]
        rc = oxa.oxa_ragged_prefill(q, k, v, qi, ki, o, max_qo_len=64, max_kv_len=1024,
                                    sm_scale=case.sm_scale, causal=True, lse=lse, workspace=ws)
        assert rc == oxa.OXA_OK, oxa.status_string(rc)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call("g")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("split graph: capture")
    with torch.cuda.graph(g):
        call("g")
    torch.cuda.synchronize()
    rng = np.random.default_rng(4605)
    for rep in range(3):
        q.copy_(dev(W.bf16_normal(rng, case.q.shape)))
        v.copy_(dev(W.bf16_normal(rng, case.v.shape)))
        note(f"split graph: replay {rep}")
        g.replay()
        call("e")
        torch.cuda.synchronize()
        assert torch.equal(outs["g"][0], outs["e"][0]), f"replay {rep} differs from eager"
        assert torch.equal(outs["g"][1], outs["e"][1])
    # the last replay against the oracle
    c2 = dataclasses.replace(case, q=host_bits(q), v=host_bits(v))
    check_ragged(c2, outs["g"][0], outs["g"][1])
