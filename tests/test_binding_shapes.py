"""The Python binding checks every tensor whose size the C ABI cannot see.

The C entry points take raw pointers, so an output or a second input of the
wrong size would let a kernel write or read past its end.  The binding derives
every size from q, k or the pools and checks the other tensors against them
before any pointer is taken; these tests pass mis-shaped CPU tensors and expect
that check to raise (it fires before the "must live on the GPU" check).
"""
import pytest
import torch

import paged_attention_02_amd as oxa

SHAPE_ERR = r"has shape|slots per page|kv heads|4 dimensions|without q_in"


def bf(*shape):
    return torch.zeros(shape, dtype=torch.int16)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


B, HQ, HKV, P = 3, 8, 2, 10


def decode_kwargs(**over):
    kw = dict(q=bf(B, HQ, 128), k_pages=bf(P, 16, HKV, 128), v_pages=bf(P, 16, HKV, 128),
              page_indptr=i32(B + 1), page_indices=i32(7), seq_lens=i32(B), o=bf(B, HQ, 128),
              lse=f32(B, HQ), status=i32(B))
    kw.update(over)
    return kw


def call_decode(**over):
    kw = decode_kwargs(**over)
    return oxa.oxa_paged_decode(kw.pop("q"), kw.pop("k_pages"), kw.pop("v_pages"),
                                kw.pop("page_indptr"), kw.pop("page_indices"),
                                kw.pop("seq_lens"), kw.pop("o"), max_seq_len=64,
                                sm_scale=0.088, **kw)


@pytest.mark.parametrize("over", [
    dict(o=bf(B, HQ, 64)),
    dict(o=bf(B + 1, HQ, 128)),
    dict(lse=f32(B, HQ + 1)),
    dict(status=i32(B + 1)),
    dict(seq_lens=i32(B - 1)),
    dict(page_indptr=i32(B)),
    dict(v_pages=bf(P - 1, 16, HKV, 128)),
    dict(k_pages=bf(P, 8, HKV, 128), v_pages=bf(P, 8, HKV, 128)),
    dict(k_pages=bf(P, 16 * HKV, 128), v_pages=bf(P, 16 * HKV, 128)),
])
def test_decode_rejects_mis_shaped_tensors(over):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        call_decode(**over)


def test_decode_checks_kv_heads_against_the_pool():
    with pytest.raises(ValueError, match=SHAPE_ERR):
        call_decode(num_kv_heads=4)


def test_decode_hnd_pool_shape():
    # an NHD-shaped pool passed as HND has 2 slots per page here
    with pytest.raises(ValueError, match=SHAPE_ERR):
        call_decode(layout="HND")


NQ, NKV = 40, 50


def ragged_call(**over):
    kw = dict(q=bf(NQ, HQ, 128), k=bf(NKV, HKV, 128), v=bf(NKV, HKV, 128), qo_indptr=i32(B + 1),
              kv_indptr=i32(B + 1), o=bf(NQ, HQ, 128), lse=f32(NQ, HQ), status=i32(B))
    kw.update(over)
    return oxa.oxa_ragged_prefill(kw.pop("q"), kw.pop("k"), kw.pop("v"), kw.pop("qo_indptr"),
                                  kw.pop("kv_indptr"), kw.pop("o"), max_qo_len=20,
                                  max_kv_len=20, sm_scale=0.088, **kw)


@pytest.mark.parametrize("over", [
    dict(o=bf(NQ - 1, HQ, 128)),
    dict(v=bf(NKV, HKV + 1, 128)),
    dict(lse=f32(NQ, 1)),
    dict(status=i32(B + 2)),
    dict(kv_indptr=i32(B)),
])
def test_ragged_prefill_rejects_mis_shaped_tensors(over):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        ragged_call(**over)


def paged_call(**over):
    kw = dict(q=bf(NQ, HQ, 128), qo_indptr=i32(B + 1), k_pages=bf(P, 16, HKV, 128),
              v_pages=bf(P, 16, HKV, 128), page_indptr=i32(B + 1), page_indices=i32(7),
              seq_lens=i32(B), o=bf(NQ, HQ, 128), lse=f32(NQ, HQ), status=i32(B))
    kw.update(over)
    return oxa.oxa_paged_prefill(kw.pop("q"), kw.pop("qo_indptr"), kw.pop("k_pages"),
                                 kw.pop("v_pages"), kw.pop("page_indptr"), kw.pop("page_indices"),
                                 kw.pop("seq_lens"), kw.pop("o"), max_qo_len=20, max_seq_len=20,
                                 sm_scale=0.088, **kw)


@pytest.mark.parametrize("over", [
    dict(o=bf(NQ, HQ, 127)),
    dict(v_pages=bf(P, 16, HKV, 64)),
    dict(lse=f32(NQ + 1, HQ)),
    dict(status=i32(1)),
    dict(seq_lens=i32(B + 1)),
    dict(page_indptr=i32(B + 2)),
])
def test_paged_prefill_rejects_mis_shaped_tensors(over):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        paged_call(**over)


T = 12


def append_call(rope, **over):
    kw = dict(q_in=bf(T, HQ, 128), q_out=bf(T, HQ, 128), k_in=bf(T, HKV, 128),
              v_in=bf(T, HKV, 128), batch_indices=i32(T), positions=i32(T),
              k_pages=bf(P, 16, HKV, 128), v_pages=bf(P, 16, HKV, 128), page_indptr=i32(B + 1),
              page_indices=i32(7), page_refcounts=i32(P), status=i32(2))
    kw.update(over)
    if rope:
        return oxa.oxa_paged_append_rope(**kw)
    kw.pop("q_in")
    kw.pop("q_out")
    return oxa.oxa_paged_append(**kw)


@pytest.mark.parametrize("rope", [True, False])
@pytest.mark.parametrize("over", [
    dict(v_in=bf(T - 1, HKV, 128)),
    dict(batch_indices=i32(T + 1)),
    dict(positions=i32(T - 1)),
    dict(v_pages=bf(P, 16, HKV, 128 * 2)),
    dict(k_pages=bf(P, 16, HKV + 2, 128), v_pages=bf(P, 16, HKV + 2, 128)),
    dict(page_refcounts=i32(P - 1)),
    dict(status=i32(1)),
])
def test_append_rejects_mis_shaped_tensors(rope, over):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        append_call(rope, **over)


@pytest.mark.parametrize("over", [
    dict(q_out=bf(T, HQ, 64)),
    dict(q_in=bf(T + 1, HQ, 128), q_out=bf(T + 1, HQ, 128)),
    dict(q_in=None),
])
def test_fused_append_rejects_mis_shaped_q(over):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        append_call(True, **over)
