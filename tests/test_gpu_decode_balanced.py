"""The load-balanced decode mode at the sizes and shapes its own code paths need.

The parametrized suite in test_gpu_decode.py runs every decode case in both
modes; this file adds what those cases cannot reach:

* page ranges of more than one 512-page descriptor window (millions of
  tokens), checked against the zero-scale closed form - every weight equal,
  so o is the mean of the sequence's V rows and lse = ln(seq_len) - computed
  in float64 on the device from the same pool (an identity of the softmax,
  not a re-implementation of the kernel);
* one workspace reused by calls of different shapes;
* 32 q heads per kv head with 8 kv heads, where each wave owns two head tiles
  and the waves run independently.
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


def a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("hq,hkv,P", [(8, 8, 1), (8, 8, 4), (32, 1, 1)])
def test_ranges_longer_than_one_window_zero_scale(hq, hkv, P):
    """One sequence of 2.2M tokens: 137,500 pages over 256 ranges of ~537 pages,
    each more than one 512-page window; the unit is cut into 256 pieces."""
    ensure_built()
    L = 2_200_000
    pages = -(-L // 16)
    g = torch.Generator(device="cuda").manual_seed(777 + hq + P)
    note(f"balanced window crossing hq={hq} hkv={hkv} P={P}: pool of {pages} pages")
    kp = torch.randn(pages, 16, hkv, 128, device="cuda", generator=g).to(torch.bfloat16)
    vp = torch.randn(pages, 16, hkv, 128, device="cuda", generator=g).to(torch.bfloat16)
    perm = torch.randperm(pages, device="cuda", generator=g).to(torch.int32)
    indptr = torch.tensor([0, pages], dtype=torch.int32, device="cuda")
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    q = torch.randn(1, hq, 128, device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(1, hq, dtype=torch.float32, device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    nb = oxa.oxa_paged_decode_balanced_workspace_bytes(1, hq, P)
    ws8 = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    rc = oxa.oxa_paged_decode(q.view(torch.int16), kp.view(torch.int16), vp.view(torch.int16),
                              indptr, perm, lens, o.view(torch.int16), max_seq_len=L,
                              sm_scale=0.0, num_kv_heads=hkv, num_partitions=P,
                              workspace=ws8.view(torch.float32), lse=lse, status=st)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    assert host(st).tolist() == [0]
    # closed form: the mean of the sequence's V rows, per kv head, in float64
    rows = vp[perm.long()].reshape(pages * 16, hkv, 128)[:L]
    mean = rows.double().mean(dim=0)                                   # [hkv, 128]
    ref = mean.repeat_interleave(hq // hkv, dim=0)[None].cpu().numpy()  # [1, hq, 128]
    assert_attention_close(host_bits(o.view(torch.int16)).reshape(1, hq, 128), ref,
                           f"window crossing hq={hq} hkv={hkv} P={P}")
    assert_lse_close(host(lse), np.full((1, hq), np.log(L)), "lse = ln L")


def test_one_workspace_reused_across_shapes():
    """One workspace sized for the largest call serves three calls of different
    shapes (independent waves, shared waves with partitions, independent again),
    each seeing the previous call's leftovers."""
    ensure_built()
    cases = [
        ("gqa4 mixed P=1", W.decode_case(601, batch=12, num_qo_heads=32, num_kv_heads=8,
                                          seq_len_range=(100, 3000), poison=True)),
        ("gqa4 mixed P=3", W.decode_case(602, batch=5, num_qo_heads=8, num_kv_heads=2,
                                          seq_len_range=(700, 2500), num_partitions=3,
                                          poison=True)),
        ("mha 16 P=1", W.decode_case(603, batch=9, num_qo_heads=16, num_kv_heads=16,
                                      seq_len_range=(1, 1500), poison=True, layout="HND")),
    ]
    nb = max(oxa.oxa_paged_decode_balanced_workspace_bytes(c.q.shape[0], c.q.shape[1],
                                                            c.num_partitions) for _, c in cases)
    ws8 = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    for what, case in cases:
        kv = case.kv
        B, hq, _ = case.q.shape
        P = case.num_partitions
        q = dev(case.q)
        o = torch.empty_like(q)
        lse = torch.empty(B, hq, dtype=torch.float32, device="cuda")
        st = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        note(f"balanced workspace reuse: {what}")
        rc = oxa.oxa_paged_decode(q, dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr),
                                  dev(kv.page_indices), dev(kv.seq_lens), o,
                                  max_seq_len=case.max_seq_len, sm_scale=case.sm_scale,
                                  layout=kv.layout, num_kv_heads=kv.num_kv_heads,
                                  num_partitions=P, workspace=ws8.view(torch.float32), lse=lse,
                                  status=st)
        assert rc == oxa.OXA_OK, oxa.status_string(rc)
        torch.cuda.synchronize()
        assert (host(st) == 0).all()
        o_ref, lse_ref = A.paged_decode(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                        kv.page_indices, kv.seq_lens, case.sm_scale)
        assert_attention_close(host_bits(o), o_ref, what)
        assert_lse_close(host(lse), lse_ref, what)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_two_head_tiles_per_wave_independent(layout):
    """256 q heads on 8 kv heads: 32 per kv head, two 16-head tiles per wave,
    8 such sets per work-group."""
    ensure_built()
    lens = [3, 16, 700, 1200, 64, 2049]
    case = W.decode_case(611, batch=len(lens), num_qo_heads=256, num_kv_heads=8, seq_lens=lens,
                         layout=layout, poison=True)
    kv = case.kv
    B, hq, _ = case.q.shape
    nb = oxa.oxa_paged_decode_balanced_workspace_bytes(B, hq, 1)
    ws8 = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    q = dev(case.q)
    o = torch.empty_like(q)
    lse = torch.empty(B, hq, dtype=torch.float32, device="cuda")
    st = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    note(f"balanced 32 q heads per kv head, 8 kv heads, {layout}")
    rc = oxa.oxa_paged_decode(q, dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr),
                              dev(kv.page_indices), dev(kv.seq_lens), o,
                              max_seq_len=case.max_seq_len, sm_scale=case.sm_scale,
                              layout=kv.layout, num_kv_heads=kv.num_kv_heads, num_partitions=1,
                              workspace=ws8.view(torch.float32), lse=lse, status=st)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    assert (host(st) == 0).all()
    o_ref, lse_ref = A.paged_decode(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                    kv.page_indices, kv.seq_lens, case.sm_scale)
    assert_attention_close(host_bits(o), o_ref, f"256/8 {layout}")
    assert_lse_close(host(lse), lse_ref)
