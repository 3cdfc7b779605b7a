"""The allocation-free paged decode (oxa_paged_decode_noalloc) gives the same
results as oxa_paged_decode with a caller workspace.

Both run the same kernels over the same partitions, so their outputs, lse and
status must agree bit for bit; both are also checked against the FP64 oracle.
Two split calls in a row share the library's static scratch - the long MQA
split-K workload first, then a smaller mixed-length GQA call - so the second
must not see anything the first left behind.  An unsplit call and a call over
the scratch limit (rejected, nothing written) close the sequence.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_helpers import assert_attention_close, assert_lse_close, dev, host, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu


def both(case, P):
    ensure_built()
    kv = case.kv
    B, hq, _ = case.q.shape
    q = dev(case.q)
    args = (dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr), dev(kv.page_indices),
            dev(kv.seq_lens))
    kw = dict(max_seq_len=case.max_seq_len, sm_scale=case.sm_scale, layout=kv.layout,
              num_kv_heads=kv.num_kv_heads, num_partitions=P)
    out = {}
    for name in ("workspace", "noalloc"):
        o = torch.full_like(q, 0x7FC0)
        lse = torch.full((B, hq), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        if name == "workspace":
            nb = oxa.oxa_paged_decode_workspace_bytes(B, hq, P)
            ws = torch.empty(max(nb, 16) // 4, dtype=torch.float32, device="cuda") if nb else None
            rc = oxa.oxa_paged_decode(q, *args, o, workspace=ws, lse=lse, status=st, **kw)
        else:
            rc = oxa.oxa_paged_decode_noalloc(q, *args, o, lse=lse, status=st, **kw)
        assert rc == oxa.OXA_OK, oxa.status_string(rc)
        torch.cuda.synchronize()
        out[name] = (host_bits(o), host(lse), host(st))
    return out


def check(case, P, what):
    note(f"noalloc decode: {what}")
    out = both(case, P)
    (o_w, l_w, s_w), (o_n, l_n, s_n) = out["workspace"], out["noalloc"]
    assert (s_n == 0).all() and np.array_equal(s_w, s_n)
    assert np.array_equal(o_w, o_n), f"{what}: o differs from oxa_paged_decode"
    assert np.array_equal(l_w.view(np.uint32), l_n.view(np.uint32)), f"{what}: lse differs"
    kv = case.kv
    o_ref, lse_ref = A.paged_decode(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                    kv.page_indices, kv.seq_lens, case.sm_scale)
    assert_attention_close(o_n, o_ref, what)
    assert_lse_close(l_n, lse_ref, what)


def test_noalloc_decode_equals_workspace_decode_on_consecutive_calls():
    # 1) the long MQA split-K workload: 8 x 32768 tokens, 32 q / 1 kv head, 16 partitions
    check(W.decode_mqa_long(), 16, "long MQA, 16 partitions")
    # 2) a smaller call right after it, reusing the scratch: mixed lengths, GQA4, HND
    lens = [1, 15, 17, 300, 2049]
    small = W.decode_case(5200, batch=len(lens), num_qo_heads=16, num_kv_heads=4, seq_lens=lens,
                          num_pages=sum(-(-n // 16) for n in lens) + 5, layout="HND",
                          poison=True)
    check(small, 3, "small GQA4 HND, 3 partitions")
    # 3) unsplit: no scratch at all
    check(small, 1, "small GQA4 HND, unsplit")


def test_noalloc_decode_over_the_limit_writes_nothing():
    ensure_built()
    case = W.decode_case(5201, batch=128, num_qo_heads=8, num_kv_heads=2, seq_lens=[40] * 128)
    kv = case.kv
    q = dev(case.q)
    o = torch.full_like(q, 0x1234)
    assert oxa.oxa_paged_decode_workspace_bytes(128, 8, 16) > oxa.OXA_DECODE_SCRATCH_BYTES
    note("noalloc decode: over the scratch limit")
    rc = oxa.oxa_paged_decode_noalloc(q, dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr),
                                      dev(kv.page_indices), dev(kv.seq_lens), o,
                                      max_seq_len=40, sm_scale=case.sm_scale, num_kv_heads=2,
                                      num_partitions=16)
    assert rc == oxa.OXA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert (o == 0x1234).all()
