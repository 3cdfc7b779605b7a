"""Attention shapes printed in the Oxide Infer README, Performance snapshot,
on the GPU vs the FP64 oracle.

Paged decode B1 / KV1 (MHA; o equals the single V row), ragged causal prefill MHA Q16 / KV16, and ragged
and paged causal prefill GQA4 with queries 32 + 64 at the end of keys
256 + 1024 (bottom-right causal alignment, fewer queries than keys).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import bf16
from tests.gpu_helpers import assert_attention_close, assert_lse_close, dev, host, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_decode_b1_kv1_returns_the_single_v_row(layout):
    case = W.pages_decode_b1_kv1(layout=layout, poison=True)
    ensure_built()
    kv = case.kv
    q = dev(case.q)
    o = torch.empty_like(q)
    lse = torch.empty(1, case.num_qo_heads, dtype=torch.float32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    note(f"pages decode B1/KV1 {layout}")
    rc = oxa.oxa_paged_decode(q, dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr),
                              dev(kv.page_indices), dev(kv.seq_lens), o, max_seq_len=1,
                              sm_scale=case.sm_scale, layout=layout, num_kv_heads=kv.num_kv_heads,
                              lse=lse, status=status)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert host(status).tolist() == [0]
    # one key: softmax weight 1, so o is that key's V row exactly (in value:
    # the accumulator starts at +0, so a -0 element comes out as +0)
    page = int(kv.page_indices[0])
    vrow = kv.v_pool[page, 0] if layout == "NHD" else kv.v_pool[page, :, 0]
    assert np.array_equal(bf16.to_f64(host_bits(o)[0]), bf16.to_f64(vrow))
    o_ref, lse_ref = A.paged_decode(case.q, kv.k_pool, kv.v_pool, layout, kv.page_indptr,
                                    kv.page_indices, kv.seq_lens, case.sm_scale)
    assert_lse_close(host(lse), lse_ref)


@pytest.mark.parametrize("which", ["mha_q16", "gqa4_32_64"])
def test_ragged_prefill_printed_shapes(which):
    case = W.pages_ragged_mha_q16() if which == "mha_q16" else W.pages_ragged_gqa4()
    ensure_built()
    q = dev(case.q)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    B = len(case.qo_indptr) - 1
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    note(f"pages ragged prefill {which}")
    rc = oxa.oxa_ragged_prefill(q, dev(case.k), dev(case.v), dev(case.qo_indptr),
                                dev(case.kv_indptr), o,
                                max_qo_len=int(np.diff(case.qo_indptr).max()),
                                max_kv_len=int(np.diff(case.kv_indptr).max()),
                                sm_scale=case.sm_scale, causal=True, lse=lse, status=status)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert (host(status) == 0).all()
    o_ref, lse_ref = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                                      case.sm_scale, True)
    assert_attention_close(host_bits(o), o_ref, which)
    assert_lse_close(host(lse), lse_ref)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_paged_prefill_gqa4_printed_shape(layout):
    case = W.pages_paged_gqa4(layout=layout, poison=True)
    ensure_built()
    kv = case.kv
    q = dev(case.q)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    status = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    note(f"pages paged prefill gqa4 {layout}")
    rc = oxa.oxa_paged_prefill(q, dev(case.qo_indptr), dev(kv.k_pool), dev(kv.v_pool),
                               dev(kv.page_indptr), dev(kv.page_indices), dev(kv.seq_lens), o,
                               max_qo_len=64, max_seq_len=1024, sm_scale=case.sm_scale,
                               layout=layout, num_kv_heads=kv.num_kv_heads, causal=True, lse=lse,
                               status=status)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert host(status).tolist() == [0, 0]
    o_ref, lse_ref = A.paged_prefill(case.q, case.qo_indptr, kv.k_pool, kv.v_pool, layout,
                                     kv.page_indptr, kv.page_indices, kv.seq_lens,
                                     case.sm_scale, True)
    assert_attention_close(host_bits(o), o_ref, f"paged gqa4 {layout}")
    assert_lse_close(host(lse), lse_ref)
    # the same keys packed contiguously through the ragged path give the same bits
    def rows(pool, b, n):
        j = np.arange(n)
        page = kv.page_indices[kv.page_indptr[b] + j // 16]
        return pool[page, j % 16] if layout == "NHD" else pool[page, :, j % 16]
    k_r = np.concatenate([rows(kv.k_pool, b, int(kv.seq_lens[b])) for b in range(2)])
    v_r = np.concatenate([rows(kv.v_pool, b, int(kv.seq_lens[b])) for b in range(2)])
    kv_indptr = np.array([0, 256, 1280], np.int32)
    o2 = torch.zeros_like(q)
    rc = oxa.oxa_ragged_prefill(q, dev(k_r), dev(v_r), dev(case.qo_indptr), dev(kv_indptr), o2,
                                max_qo_len=64, max_kv_len=1024, sm_scale=case.sm_scale,
                                causal=True)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o2), host_bits(o)), "paged and ragged paths disagree"
