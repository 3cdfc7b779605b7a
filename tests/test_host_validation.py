"""Host-side contract checks of the C ABI: each call below breaks one rule and
must return the matching OXA_ERR_* code before touching the GPU.

The pointers are fake (never dereferenced): validation rejects the call first.
These tests do not run where a GPU is visible, so a validation bug can never
turn one of them into a real launch.
"""
import pytest
import torch

from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake-pointer validation tests run on GPU-less hosts only")

A = 1 << 32          # a 16-byte aligned fake address space, regions far apart
GAP = 1 << 30


def addr(i):
    return A + i * GAP


def decode_args(**over):
    args = dict(stream=None, q=addr(0), batch=2, hq=8, hkv=2, head_dim=128, k=addr(1), v=addr(2),
                num_pages=10, page_size=16, layout=0, indptr=addr(3), indices=addr(4),
                num_entries=6, seq_lens=addr(5), max_seq_len=64, scale=0.088, P=1,
                ws=None, ws_bytes=0, o=addr(6), lse=None, status=None)
    args.update(over)
    return list(args.values())


def call_decode(**over):
    return ensure_built().oxa_paged_decode(*decode_args(**over))


@pytest.mark.parametrize("over,code", [
    (dict(q=None), oxa.OXA_ERR_NULL),
    (dict(o=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=64), oxa.OXA_ERR_UNSUPPORTED),
    (dict(page_size=32), oxa.OXA_ERR_UNSUPPORTED),
    (dict(layout=2), oxa.OXA_ERR_UNSUPPORTED),
    (dict(hq=6, hkv=4), oxa.OXA_ERR_SHAPE),
    (dict(batch=0), oxa.OXA_ERR_SHAPE),
    (dict(max_seq_len=0), oxa.OXA_ERR_SHAPE),
    (dict(P=0), oxa.OXA_ERR_SHAPE),
    (dict(P=1025), oxa.OXA_ERR_SHAPE),
    (dict(num_pages=0), oxa.OXA_ERR_SHAPE),
    (dict(scale=float("nan")), oxa.OXA_ERR_SHAPE),
    (dict(scale=-0.5), oxa.OXA_ERR_SHAPE),
    (dict(q=addr(0) + 8), oxa.OXA_ERR_ALIGN),
    (dict(seq_lens=addr(5) + 2), oxa.OXA_ERR_ALIGN),
    (dict(P=4), oxa.OXA_ERR_WORKSPACE),
    (dict(P=4, ws=addr(7), ws_bytes=100), oxa.OXA_ERR_WORKSPACE),
    (dict(o=addr(0) + 512), oxa.OXA_ERR_ALIAS),            # o overlaps q
    (dict(lse=addr(1) + 4096), oxa.OXA_ERR_ALIAS),         # lse inside the K pool
    (dict(status=addr(6) + 16), oxa.OXA_ERR_ALIAS),        # status inside o
    (dict(P=4, ws=addr(2), ws_bytes=1 << 20), oxa.OXA_ERR_ALIAS),  # workspace over the V pool
])
def test_decode_rejections(over, code):
    assert call_decode(**over) == code


def call_decode_noalloc(**over):
    args = decode_args(**over)
    del args[18:20]  # the allocation-free form takes no workspace arguments
    return ensure_built().oxa_paged_decode_noalloc(*args)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=64), oxa.OXA_ERR_UNSUPPORTED),
    (dict(P=0), oxa.OXA_ERR_SHAPE),
    (dict(scale=-0.5), oxa.OXA_ERR_SHAPE),
    (dict(q=addr(0) + 8), oxa.OXA_ERR_ALIGN),
    (dict(o=addr(0) + 512), oxa.OXA_ERR_ALIAS),
    # partial states of 128 x 8 x 16 (row, partition) pairs: 8,454,144 bytes > 8 MiB
    (dict(batch=128, hq=8, P=16), oxa.OXA_ERR_SCRATCH_LIMIT),
    (dict(batch=16, hq=8, P=128), oxa.OXA_ERR_SCRATCH_LIMIT),
])
def test_decode_noalloc_rejections(over, code):
    assert call_decode_noalloc(**over) == code


def test_decode_noalloc_limit_matches_the_workspace_query():
    limit = oxa.OXA_DECODE_SCRATCH_BYTES
    assert oxa.oxa_paged_decode_workspace_bytes(127, 8, 16) <= limit   # 16256 states fit
    assert oxa.oxa_paged_decode_workspace_bytes(128, 8, 16) > limit


def call_ragged(**over):
    args = dict(stream=None, q=addr(0), k=addr(1), v=addr(2), qo=addr(3), kv=addr(4), batch=2,
                nnz_qo=100, nnz_kv=100, hq=8, hkv=2, head_dim=128, max_qo=64, max_kv=64,
                causal=1, scale=0.088, ws=None, ws_bytes=0, o=addr(5), lse=None, status=None)
    args.update(over)
    return ensure_built().oxa_ragged_prefill(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(k=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=256), oxa.OXA_ERR_UNSUPPORTED),
    (dict(hq=8, hkv=3), oxa.OXA_ERR_SHAPE),
    (dict(nnz_qo=-1), oxa.OXA_ERR_SHAPE),
    (dict(max_qo=0), oxa.OXA_ERR_SHAPE),
    (dict(scale=float("-inf")), oxa.OXA_ERR_SHAPE),
    (dict(max_qo=1 << 30), oxa.OXA_ERR_SHAPE),       # more query tiles than the grid allows
    (dict(hq=256, hkv=1, max_qo=4097), oxa.OXA_ERR_SHAPE),  # one-row tiles: at most 4096 levels
    (dict(v=addr(2) + 4), oxa.OXA_ERR_ALIGN),
    (dict(o=addr(1) + 256), oxa.OXA_ERR_ALIAS),      # o overlaps k
    (dict(status=addr(4)), oxa.OXA_ERR_ALIAS),       # status over kv_indptr
    (dict(ws=addr(8) + 4, ws_bytes=1 << 24), oxa.OXA_ERR_ALIGN),
    (dict(ws=addr(8), ws_bytes=8 * 100 * 8 * 516 - 1), oxa.OXA_ERR_WORKSPACE),
    (dict(ws=addr(5) - 4096, ws_bytes=1 << 24), oxa.OXA_ERR_ALIAS),    # runs into o
    (dict(ws=addr(0), ws_bytes=1 << 24), oxa.OXA_ERR_ALIAS),           # over q
])
def test_ragged_rejections(over, code):
    assert call_ragged(**over) == code


def call_paged_prefill(**over):
    args = dict(stream=None, q=addr(0), qo=addr(1), k=addr(2), v=addr(3), num_pages=10,
                page_size=16, layout=1, indptr=addr(4), indices=addr(5), num_entries=10,
                seq_lens=addr(6), batch=2, nnz_qo=50, hq=4, hkv=4, head_dim=128, max_qo=64,
                max_seq=64, causal=1, scale=0.088, ws=None, ws_bytes=0, o=addr(7), lse=None,
                status=None)
    args.update(over)
    return ensure_built().oxa_paged_prefill(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(seq_lens=None), oxa.OXA_ERR_NULL),
    (dict(layout=-1), oxa.OXA_ERR_UNSUPPORTED),
    (dict(num_entries=-1), oxa.OXA_ERR_SHAPE),
    (dict(max_seq=0), oxa.OXA_ERR_SHAPE),
    (dict(o=addr(7) + 2), oxa.OXA_ERR_ALIGN),
    (dict(lse=addr(3) + 8), oxa.OXA_ERR_ALIAS),
    (dict(ws=addr(9) + 8, ws_bytes=1 << 24), oxa.OXA_ERR_ALIGN),
    (dict(ws=addr(9), ws_bytes=8 * 50 * 4 * 516 - 4), oxa.OXA_ERR_WORKSPACE),
    (dict(ws=addr(7), ws_bytes=1 << 24), oxa.OXA_ERR_ALIAS),           # over o
])
def test_paged_prefill_rejections(over, code):
    assert call_paged_prefill(**over) == code


def call_append(**over):
    args = dict(stream=None, q_in=addr(0), q_out=addr(1), hq=8, k_in=addr(2), v_in=addr(3), hkv=2,
                head_dim=128, bidx=addr(4), pos=addr(5), nnz=20, kp=addr(6), vp=addr(7),
                num_pages=10, page_size=16, layout=0, indptr=addr(8), batch=2, indices=addr(9),
                num_entries=10, refc=addr(10), theta=10000.0, ws=addr(12), ws_bytes=8192,
                status=addr(11))
    args.update(over)
    return ensure_built().oxa_paged_append_rope(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(status=None), oxa.OXA_ERR_NULL),
    (dict(refc=None), oxa.OXA_ERR_NULL),
    (dict(q_out=None), oxa.OXA_ERR_NULL),               # q_in without q_out
    (dict(head_dim=96), oxa.OXA_ERR_UNSUPPORTED),
    (dict(page_size=8), oxa.OXA_ERR_UNSUPPORTED),
    (dict(nnz=-3), oxa.OXA_ERR_SHAPE),
    (dict(batch=0), oxa.OXA_ERR_SHAPE),
    (dict(theta=0.0), oxa.OXA_ERR_SHAPE),
    (dict(theta=float("inf")), oxa.OXA_ERR_SHAPE),
    (dict(k_in=addr(2) + 8), oxa.OXA_ERR_ALIGN),
    (dict(pos=addr(5) + 1), oxa.OXA_ERR_ALIGN),
    (dict(q_out=addr(0) + 256), oxa.OXA_ERR_ALIAS),     # partial overlap with q_in
    (dict(kp=addr(2)), oxa.OXA_ERR_ALIAS),              # K pool over k_in
    (dict(status=addr(6) + 64), oxa.OXA_ERR_ALIAS),     # status inside the K pool
    (dict(ws=None), oxa.OXA_ERR_WORKSPACE),
    (dict(ws_bytes=8191), oxa.OXA_ERR_WORKSPACE),
    (dict(ws=addr(12) + 8), oxa.OXA_ERR_ALIGN),
    (dict(ws=addr(7) + 4096), oxa.OXA_ERR_ALIAS),       # workspace inside the V pool
    (dict(vp=addr(6) + 1024), oxa.OXA_ERR_ALIAS),       # V pool overlaps K pool
])
def test_append_rejections(over, code):
    assert call_append(**over) == code


def call_plain_append(**over):
    args = dict(stream=None, k_in=addr(2), v_in=addr(3), hkv=2, head_dim=128, bidx=addr(4),
                pos=addr(5), nnz=20, kp=addr(6), vp=addr(7), num_pages=10, page_size=16,
                layout=1, indptr=addr(8), batch=2, indices=addr(9), num_entries=10,
                refc=addr(10), ws=addr(12), ws_bytes=8192, status=addr(11))
    args.update(over)
    return ensure_built().oxa_paged_append(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(status=None), oxa.OXA_ERR_NULL),
    (dict(v_in=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=64), oxa.OXA_ERR_UNSUPPORTED),
    (dict(layout=2), oxa.OXA_ERR_UNSUPPORTED),
    (dict(hkv=0), oxa.OXA_ERR_SHAPE),
    (dict(batch=0), oxa.OXA_ERR_SHAPE),
    (dict(v_in=addr(3) + 4), oxa.OXA_ERR_ALIGN),
    (dict(kp=addr(3)), oxa.OXA_ERR_ALIAS),              # K pool over v_in
    (dict(ws_bytes=100), oxa.OXA_ERR_WORKSPACE),
    (dict(ws=addr(6) + 512), oxa.OXA_ERR_ALIAS),        # workspace inside the K pool
])
def test_plain_append_rejections(over, code):
    assert call_plain_append(**over) == code


def call_merge(**over):
    args = dict(stream=None, v=addr(0), lse=addr(1), v_dtype=0, rows=4, states=3, heads=8,
                head_dim=128, v_out=addr(2), out_dtype=0, lse_out=addr(3))
    args.update(over)
    return ensure_built().oxa_merge_states(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(v=None), oxa.OXA_ERR_NULL),
    (dict(lse=None), oxa.OXA_ERR_NULL),
    (dict(v_out=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=64), oxa.OXA_ERR_UNSUPPORTED),
    (dict(v_dtype=2), oxa.OXA_ERR_UNSUPPORTED),
    (dict(out_dtype=-1), oxa.OXA_ERR_UNSUPPORTED),
    (dict(rows=-1), oxa.OXA_ERR_SHAPE),
    (dict(states=0), oxa.OXA_ERR_SHAPE),
    (dict(heads=0), oxa.OXA_ERR_SHAPE),
    (dict(v=addr(0) + 8), oxa.OXA_ERR_ALIGN),
    (dict(v_out=addr(2) + 4), oxa.OXA_ERR_ALIGN),
    (dict(lse_out=addr(3) + 2), oxa.OXA_ERR_ALIGN),
    (dict(v_out=addr(0) + 1024), oxa.OXA_ERR_ALIAS),    # output inside the states
    (dict(lse_out=addr(1) + 16), oxa.OXA_ERR_ALIAS),    # lse_out inside lse
    (dict(lse_out=addr(2) + 256), oxa.OXA_ERR_ALIAS),   # lse_out inside v_out
    (dict(v_out=addr(0)), oxa.OXA_ERR_ALIAS),           # no in-place form for S states
])
def test_merge_states_rejections(over, code):
    assert call_merge(**over) == code


def test_merge_with_no_rows_is_a_no_op():
    # nothing to merge: accepted without pointers, nothing enqueued
    assert call_merge(rows=0, v=None, lse=None, v_out=None, lse_out=None) == oxa.OXA_OK


def call_pair(**over):
    args = dict(stream=None, v_a=addr(0), lse_a=addr(1), v_b=addr(2), lse_b=addr(3), v_dtype=0,
                rows=4, heads=8, head_dim=128, v_out=addr(4), out_dtype=0, lse_out=addr(5))
    args.update(over)
    return ensure_built().oxa_merge_state_pair(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(v_b=None), oxa.OXA_ERR_NULL),
    (dict(lse_b=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=256), oxa.OXA_ERR_UNSUPPORTED),
    (dict(v_dtype=7), oxa.OXA_ERR_UNSUPPORTED),
    (dict(rows=-2), oxa.OXA_ERR_SHAPE),
    (dict(heads=0), oxa.OXA_ERR_SHAPE),
    (dict(v_b=addr(2) + 2), oxa.OXA_ERR_ALIGN),
    (dict(lse_a=addr(1) + 1), oxa.OXA_ERR_ALIGN),
    (dict(v_out=addr(0) + 256), oxa.OXA_ERR_ALIAS),     # partial overlap with v_a
    (dict(v_out=addr(0), out_dtype=1), oxa.OXA_ERR_ALIAS),  # in place needs one dtype
    (dict(lse_out=addr(1) + 4), oxa.OXA_ERR_ALIAS),     # shifted onto lse_a
    (dict(lse_out=addr(2)), oxa.OXA_ERR_ALIAS),         # lse_out over v_b
    (dict(v_out=addr(3)), oxa.OXA_ERR_ALIAS),           # v_out over lse_b
])
def test_merge_state_pair_rejections(over, code):
    assert call_pair(**over) == code


def call_rope(llama=False, **over):
    args = dict(stream=None, q_in=addr(0), q_out=addr(1), hq=8, k_in=addr(2), k_out=addr(3),
                hkv=2, head_dim=128, pos=addr(4), nnz=10, theta=10000.0)
    extra = dict(factor=8.0, low=1.0, high=4.0, orig=8192)
    args.update({k: v for k, v in over.items() if k in args})
    extra.update({k: v for k, v in over.items() if k in extra})
    lib = ensure_built()
    if llama:
        return lib.oxa_rope_llama31(*args.values(), *extra.values())
    return lib.oxa_rope_neox(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q_out=None), oxa.OXA_ERR_NULL),                 # q_in without q_out
    (dict(k_in=None), oxa.OXA_ERR_NULL),                  # k_out without k_in
    (dict(pos=None), oxa.OXA_ERR_NULL),
    (dict(q_in=None, q_out=None, k_in=None, k_out=None), oxa.OXA_ERR_NULL),
    (dict(head_dim=64), oxa.OXA_ERR_UNSUPPORTED),
    (dict(nnz=-1), oxa.OXA_ERR_SHAPE),
    (dict(hq=0), oxa.OXA_ERR_SHAPE),
    (dict(theta=-1.0), oxa.OXA_ERR_SHAPE),
    (dict(theta=float("nan")), oxa.OXA_ERR_SHAPE),
    (dict(k_out=addr(3) + 8), oxa.OXA_ERR_ALIGN),
    (dict(pos=addr(4) + 2), oxa.OXA_ERR_ALIGN),
    (dict(q_out=addr(0) + 256), oxa.OXA_ERR_ALIAS),       # shifted onto q_in
    (dict(k_out=addr(1)), oxa.OXA_ERR_ALIAS),             # k_out over q_out
    (dict(q_out=addr(2)), oxa.OXA_ERR_ALIAS),             # q_out over k_in
    (dict(pos=addr(3) + 64), oxa.OXA_ERR_ALIAS),          # positions inside k_out
])
def test_rope_rejections(over, code):
    assert call_rope(**over) == code


@pytest.mark.parametrize("over,code", [
    (dict(factor=0.0), oxa.OXA_ERR_SHAPE),
    (dict(low=0.0), oxa.OXA_ERR_SHAPE),
    (dict(high=1.0), oxa.OXA_ERR_SHAPE),                 # high must exceed low
    (dict(orig=0), oxa.OXA_ERR_SHAPE),
    (dict(factor=float("inf")), oxa.OXA_ERR_SHAPE),
    (dict(theta=0.0), oxa.OXA_ERR_SHAPE),
    (dict(pos=None), oxa.OXA_ERR_NULL),
])
def test_rope_llama31_rejections(over, code):
    assert call_rope(llama=True, **over) == code


def test_rope_with_no_tokens_is_a_no_op():
    assert call_rope(nnz=0, q_in=None, q_out=None, k_in=None, k_out=None, pos=None) == oxa.OXA_OK
    assert call_rope(llama=True, nnz=0, pos=None) == oxa.OXA_OK
