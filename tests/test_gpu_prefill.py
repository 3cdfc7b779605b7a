"""Ragged and paged causal prefill on the GPU vs the FP64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import rope as R
from tests.gpu_helpers import (assert_attention_close, assert_lse_close, dev, host, host_bits,
                               note)
from tests.lib_loader import ensure_built
from tests.oracle_helpers import scatter_pages

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu


def run_ragged(case, *, max_qo=None, max_kv=None):
    ensure_built()
    q = dev(case.q)
    o = torch.empty_like(q)
    o.fill_(0)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    B = len(case.qo_indptr) - 1
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    qlens = np.diff(case.qo_indptr)
    klens = np.diff(case.kv_indptr)
    rc = oxa.oxa_ragged_prefill(q, dev(case.k), dev(case.v), dev(case.qo_indptr),
                                dev(case.kv_indptr), o,
                                max_qo_len=max_qo or max(1, int(qlens.max())),
                                max_kv_len=max_kv or max(1, int(klens.max())),
                                sm_scale=case.sm_scale, causal=case.causal, lse=lse, status=status)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    return dict(o=host_bits(o), lse=host(lse), status=host(status))


def run_paged(q_bits, qo_indptr, kp, vp, layout, indptr, ids, seq_lens, hkv, scale, causal=True,
              max_qo=None, max_seq=None):
    ensure_built()
    q = dev(q_bits)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    B = len(qo_indptr) - 1
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    rc = oxa.oxa_paged_prefill(q, dev(qo_indptr), dev(kp), dev(vp), dev(indptr), dev(ids),
                               dev(np.asarray(seq_lens, np.int32)), o,
                               max_qo_len=max_qo or max(1, int(np.diff(qo_indptr).max())),
                               max_seq_len=max_seq or max(1, int(np.max(seq_lens))),
                               sm_scale=scale, layout=layout, num_kv_heads=hkv, causal=causal,
                               lse=lse, status=status)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    return dict(o=host_bits(o), lse=host(lse), status=host(status))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (2, 1), (8, 2), (32, 8), (32, 1), (12, 4), (48, 2),
                                    (64, 1), (512, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_prefill_small(hq, hkv, causal):
    lens = [1, 17, 64, 130, 300]
    case = W.ragged_case(31 + hq, qo_lens=lens, num_qo_heads=hq, num_kv_heads=hkv, causal=causal)
    note(f"ragged hq={hq} hkv={hkv} causal={causal}")
    got = run_ragged(case)
    o, lse = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                              case.sm_scale, causal)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"ragged hq={hq} hkv={hkv}")
    assert_lse_close(got["lse"], lse)


def test_ragged_prefill_fewer_queries_than_keys():
    # bottom-right causal alignment: query chunks at the end of longer key ranges
    case = W.ragged_case(40, qo_lens=[3, 70, 129], kv_lens=[50, 70, 400], num_qo_heads=8,
                         num_kv_heads=2)
    note("ragged qo<kv")
    got = run_ragged(case)
    o, lse = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                              case.sm_scale, True)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, "qo<kv")


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_paged_prefill_matches_oracle_and_ragged_bits(layout):
    lens = [1, 40, 150, 257]
    hq, hkv = 32, 8
    case = W.ragged_case(41, qo_lens=lens, num_qo_heads=hq, num_kv_heads=hkv)
    ks = [case.k[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(len(lens))]
    vs = [case.v[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(len(lens))]
    npages = sum(-(-n // 16) for n in lens) + 6
    kp, indptr, ids = scatter_pages(ks, npages, layout, np.random.default_rng(1))
    vp, _, _ = scatter_pages(vs, npages, layout, np.random.default_rng(1))
    note(f"paged prefill {layout}")
    got = run_paged(case.q, case.qo_indptr, kp, vp, layout, indptr, ids, lens, hkv,
                    case.sm_scale)
    o, lse = A.paged_prefill(case.q, case.qo_indptr, kp, vp, layout, indptr, ids, lens,
                             case.sm_scale, True)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"paged {layout}")
    assert_lse_close(got["lse"], lse)
    rag = run_ragged(case)
    assert np.array_equal(rag["o"], got["o"]), "paged and ragged paths disagree on identical data"


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_paged_prefill_non_causal_more_queries_than_keys(layout):
    """Full (non-causal) attention allows qo_len > kv_len: 100 queries over 40
    paged keys, 7 over 300, 65 over 1."""
    qo, kv = [100, 7, 65], [40, 300, 1]
    hq, hkv = 16, 4
    case = W.ragged_case(43, qo_lens=qo, kv_lens=kv, num_qo_heads=hq, num_kv_heads=hkv,
                         causal=False)
    ks = [case.k[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(3)]
    vs = [case.v[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(3)]
    npages = sum(-(-n // 16) for n in kv) + 3
    kp, indptr, ids = scatter_pages(ks, npages, layout, np.random.default_rng(3))
    vp, _, _ = scatter_pages(vs, npages, layout, np.random.default_rng(3))
    note(f"paged prefill non-causal {layout}")
    got = run_paged(case.q, case.qo_indptr, kp, vp, layout, indptr, ids, kv, hkv, case.sm_scale,
                    causal=False)
    o, lse = A.paged_prefill(case.q, case.qo_indptr, kp, vp, layout, indptr, ids,
                             np.array(kv, np.int32), case.sm_scale, False)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"paged non-causal {layout}")
    assert_lse_close(got["lse"], lse)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("split", [False, True])
def test_paged_prefill_across_page_id_windows(layout, split):
    """A sequence of 40000 keys lists 2500 pages, more than the 2048-page window
    of page ids the prefill kernel stages at a time: 64 queries at its end and
    a short second sequence, unsplit and split into 8 key chunks (with the
    workspace), the last of which starts in the second window."""
    qo, kv = [64, 5], [40000, 40]
    hq, hkv = 8, 2
    case = W.ragged_case(44, qo_lens=qo, kv_lens=kv, num_qo_heads=hq, num_kv_heads=hkv)
    ks = [case.k[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(2)]
    vs = [case.v[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(2)]
    npages = sum(-(-n // 16) for n in kv) + 5
    kp, indptr, ids = scatter_pages(ks, npages, layout, np.random.default_rng(4))
    vp, _, _ = scatter_pages(vs, npages, layout, np.random.default_rng(4))
    assert indptr[1] > 2048
    ensure_built()
    q = dev(case.q)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    status = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    ws = None
    if split:
        nb = oxa.oxa_paged_prefill_workspace_bytes(2, q.shape[0], hq)
        assert nb > 0
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    note(f"paged prefill across page-id windows {layout} split={split}")
    rc = oxa.oxa_paged_prefill(q, dev(case.qo_indptr), dev(kp), dev(vp), dev(indptr), dev(ids),
                               dev(np.array(kv, np.int32)), o, max_qo_len=64, max_seq_len=40000,
                               sm_scale=case.sm_scale, layout=layout, num_kv_heads=hkv,
                               causal=True, lse=lse, status=status, workspace=ws)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    assert host(status).tolist() == [0, 0]
    if split:
        assert (ws != 0xFF).any(), "the call did not split"
    o_ref, lse_ref = A.paged_prefill(case.q, case.qo_indptr, kp, vp, layout, indptr, ids,
                                     np.array(kv, np.int32), case.sm_scale, True)
    assert_attention_close(host_bits(o), o_ref, f"windows {layout} split={split}")
    assert_lse_close(host(lse), lse_ref)


def test_paged_prefill_status():
    lens = [40, 40, 40]
    case = W.ragged_case(42, qo_lens=lens, num_qo_heads=4, num_kv_heads=1)
    ks = [case.k[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(3)]
    kp, indptr, ids = scatter_pages(ks, 12, "NHD", np.random.default_rng(2))
    ids = ids.copy()
    ids[indptr[1] + 1] = 99                        # sequence 1: page outside the pool
    seq_lens = np.array([40, 40, 30], np.int32)    # sequence 2: 40 queries, 30 keys (causal)
    note("paged prefill status")
    got = run_paged(case.q, case.qo_indptr, kp, kp, "NHD", indptr, ids, seq_lens, 1,
                    case.sm_scale)
    assert got["status"].tolist() == [0, oxa.OXA_DEV_PAGE_RANGE, oxa.OXA_DEV_CAUSAL]
    reasons = A.paged_prefill_status(case.qo_indptr, len(case.q), seq_lens, indptr, len(ids), ids,
                                     12, 40, 40, True)
    assert reasons == [None, "page_range", "causal"]
    o, _ = A.paged_prefill(case.q[:40], case.qo_indptr[:2], kp, kp, "NHD", indptr, ids,
                           seq_lens[:1], case.sm_scale, True)
    assert_attention_close(got["o"][:40], o, "valid sequence")


def _sample_rows(qo_indptr, per_seq, rng):
    rows = []
    for b in range(len(qo_indptr) - 1):
        s, e = int(qo_indptr[b]), int(qo_indptr[b + 1])
        pick = {s, s + 1, e - 1, e - 2, s + 63, s + 64, s + 127, s + 128}
        pick |= set(rng.integers(s, e, size=per_seq).tolist())
        rows += sorted(r for r in pick if s <= r < e)
    return np.array(rows)


def _full_tile_rows(qo_indptr, tile=64):
    """Every row of whole query tiles (64 rows x the 4 q heads of a kv head in
    the GQA4 shapes): the last two tiles of each sequence (the longest causal
    level) and a tile pair in its middle, aligned to the tile grid."""
    rows = []
    for b in range(len(qo_indptr) - 1):
        s, e = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n = e - s
        mid = s + (n // 2 // tile) * tile
        pick = set(range(max(s, e - 2 * tile), e)) | set(range(mid, min(e, mid + 2 * tile)))
        rows += sorted(pick)
    return np.array(rows)


def test_ragged_prefill_full_size_sampled():
    # lengths {512, 1024, 2048, 4096}, 32 q / 8 kv heads, causal
    case = W.ragged_gqa4_prefill()
    note("ragged full size")
    got = run_ragged(case)
    assert (got["status"] == 0).all()
    rows = _sample_rows(case.qo_indptr, 24, np.random.default_rng(0))
    o, lse = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                              case.sm_scale, True, rows=rows)
    assert_attention_close(got["o"][rows], o[rows], "ragged full sampled")
    assert_lse_close(got["lse"][rows], lse[rows])
    # whole query tiles, all 32 heads: the last 128 rows and a mid pair per sequence
    tiles = _full_tile_rows(case.qo_indptr)
    o, lse = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                              case.sm_scale, True, rows=tiles)
    assert_attention_close(got["o"][tiles], o[tiles], "ragged full tiles")
    assert_lse_close(got["lse"][tiles], lse[tiles])


def test_rope_append_then_paged_prefill_full_size_sampled():
    # fused RoPE + append of 2 x 16384 tokens, then paged causal prefill over those pages
    case = W.rope_append_prefill()
    kv = case.kv
    ensure_built()
    q_in = dev(case.q)
    q_rot = torch.empty_like(q_in)
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    status = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    indptr, ids = dev(kv.page_indptr), dev(kv.page_indices)
    note("append + paged prefill full size")
    rc = oxa.oxa_paged_append_rope(q_in, q_rot, dev(case.k), dev(case.v),
                                   dev(case.batch_indices), dev(case.positions), kp, vp, indptr,
                                   ids, dev(case.page_refcounts), status, layout=kv.layout,
                                   rope_theta=case.rope_theta)
    assert rc == oxa.OXA_OK
    o = torch.zeros_like(q_in)
    lse = torch.empty(q_in.shape[0], q_in.shape[1], dtype=torch.float32, device="cuda")
    st2 = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    rc = oxa.oxa_paged_prefill(q_rot, dev(case.qo_indptr), kp, vp, indptr, ids,
                               dev(kv.seq_lens), o, max_qo_len=16384, max_seq_len=16384,
                               sm_scale=case.sm_scale, layout=kv.layout, num_kv_heads=8,
                               causal=True, lse=lse, status=st2)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert host(status).tolist() == [0, -1] and host(st2).tolist() == [0, 0]
    # oracle: its own RoPE + append, then its paged prefill on sampled rows
    reason, q_ref, k_ref, v_ref = R.paged_append_rope(
        case.q, case.k, case.v, case.batch_indices, case.positions, kv.k_pool, kv.v_pool,
        kv.layout, kv.page_indptr, kv.page_indices, case.page_refcounts, case.rope_theta)
    assert reason is None
    rows = _sample_rows(case.qo_indptr, 12, np.random.default_rng(1))
    o_ref, _ = A.paged_prefill(q_ref, case.qo_indptr, k_ref, v_ref, kv.layout, kv.page_indptr,
                               kv.page_indices, kv.seq_lens, case.sm_scale, True, rows=rows)
    got_o, got_lse = host_bits(o), host(lse)
    assert_attention_close(got_o[rows], o_ref[rows], "paged prefill full sampled")
    # whole query tiles, all 32 heads: the last 128 rows of each 16384-row
    # sequence (the longest causal level) and a tile pair in its middle
    tiles = _full_tile_rows(case.qo_indptr)
    note(f"paged prefill full tiles: {len(tiles)} rows x 32 heads against the oracle")
    o_ref, lse_ref = A.paged_prefill(q_ref, case.qo_indptr, k_ref, v_ref, kv.layout,
                                     kv.page_indptr, kv.page_indices, kv.seq_lens, case.sm_scale,
                                     True, rows=tiles)
    assert_attention_close(got_o[tiles], o_ref[tiles], "paged prefill full tiles")
    assert_lse_close(got_lse[tiles], lse_ref[tiles])
