"""Paged decode on the GPU vs the FP64 oracle (MHA / GQA / MQA, split-K, NHD / HND)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import bf16
from tests.gpu_helpers import (assert_attention_close, assert_lse_close, dev, host, host_bits,
                               note)
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu


def a256(x):
    return (x + 255) // 256 * 256


def run_decode(case, *, num_partitions=None, with_ws_view=False, max_seq_len=None,
               mode="direct"):
    """Run oxa_paged_decode.  mode "direct": the minimal workspace; "balanced":
    the load-balanced mode's workspace, all 0xFF bytes (NaN floats) on entry,
    so a piece or partition state read before it was written shows."""
    ensure_built()
    kv = case.kv
    P = case.num_partitions if num_partitions is None else num_partitions
    B, hq, _ = case.q.shape
    msl = case.max_seq_len if max_seq_len is None else max_seq_len
    q = dev(case.q)
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    o = torch.empty_like(q)
    lse = torch.empty(B, hq, dtype=torch.float32, device="cuda")
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    state = B * hq * P * 129 * 4 if P > 1 else 0
    if mode == "balanced":
        nbytes = oxa.oxa_paged_decode_balanced_workspace_bytes(B, hq, P)
        assert nbytes > 0
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda").view(torch.float32)
    else:
        nbytes = oxa.oxa_paged_decode_workspace_bytes(B, hq, P)
        ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device="cuda") if nbytes else None
    note(f"  decode call mode={mode} B={B} hq={hq} P={P} layout={kv.layout}")
    rc = oxa.oxa_paged_decode(q, kp, vp, dev(kv.page_indptr), dev(kv.page_indices),
                              dev(kv.seq_lens), o, max_seq_len=msl, sm_scale=case.sm_scale,
                              layout=kv.layout, num_kv_heads=kv.num_kv_heads, num_partitions=P,
                              workspace=ws, lse=lse, status=status)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    torch.cuda.synchronize()
    out = dict(o=host_bits(o), lse=host(lse), status=host(status))
    if mode == "balanced":
        meta = ws.view(torch.uint8)[a256(state):][:4].view(torch.int32)
        # the balanced kernel writes the unit page starts (the first is 0)
        # whenever the call has 64 pages or more of largest possible total
        ran = meta.item() == 0
        assert ran == (B * -(-msl // 16) >= 64), "balanced mode taken iff the call is large enough"
        out["balanced_ran"] = ran
    if with_ws_view and ws is not None and P > 1:
        rows = B * hq * P
        flat = host(ws)
        out["o_part"] = flat[: rows * 128].reshape(B, hq, P, 128)
        out["lse_part"] = flat[rows * 128: rows * 129].reshape(B, hq, P)
    return out


MODES = ["direct", "balanced"]


def oracle_decode(case):
    kv = case.kv
    return A.paged_decode(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                          kv.page_indices, kv.seq_lens, case.sm_scale)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("mode", MODES)
def test_single_sequence_mha_decode(layout, mode):
    case = W.decode_mha_small(poison=True, layout=layout)
    note(f"decode mha small {layout}")
    got = run_decode(case, mode=mode)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, "mha")
    assert_lse_close(got["lse"], lse, "mha lse")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (32, 1), (64, 1), (48, 1), (12, 4), (16, 16),
                                    (1, 1)])
@pytest.mark.parametrize("P", [1, 3])
@pytest.mark.parametrize("mode", MODES)
def test_grouped_decode_mixed_lengths(hq, hkv, P, mode):
    lens = [1, 15, 16, 17, 33, 200, 531]
    case = W.decode_case(77 + hq + hkv, batch=len(lens), num_qo_heads=hq, num_kv_heads=hkv,
                         seq_lens=lens, num_pages=sum(-(-n // 16) for n in lens) + 9,
                         num_partitions=P, poison=True)
    note(f"decode grouped hq={hq} hkv={hkv} P={P}")
    got = run_decode(case, mode=mode, with_ws_view=True)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"hq={hq} hkv={hkv} P={P}")
    assert_lse_close(got["lse"], lse)
    if P > 1:
        kv = case.kv
        op, lp = A.decode_partials(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                   kv.page_indices, kv.seq_lens, case.sm_scale, P,
                                   case.max_seq_len)
        live = np.isfinite(lp)
        assert np.array_equal(np.isfinite(got["lse_part"]), live)
        np.testing.assert_allclose(got["lse_part"][live], lp[live], rtol=1e-4, atol=2e-4)
        assert not got["o_part"][~live].any()
        err = got["o_part"][live] - op[live]
        assert np.max(np.abs(err)) <= 2e-2
        assert np.linalg.norm(err) / np.linalg.norm(op[live]) <= 5e-3


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("P", [1, 2])
@pytest.mark.parametrize("mode", MODES)
def test_decode_several_head_tiles_per_kv_head(layout, P, mode):
    """24 q heads per kv head: two work-groups (16 + 8 heads, the second tile
    partly empty) read the same K/V rows, in both layouts."""
    lens = [5, 160, 1000, 47]
    case = W.decode_case(90 + P, batch=len(lens), num_qo_heads=48, num_kv_heads=2, seq_lens=lens,
                         num_pages=sum(-(-n // 16) for n in lens) + 4, layout=layout,
                         num_partitions=P, poison=True)
    note(f"decode 24 q heads per kv head {layout} P={P}")
    got = run_decode(case, mode=mode)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"24 heads per kv head {layout} P={P}")
    assert_lse_close(got["lse"], lse)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("mode", MODES)
def test_batch_gqa4_decode_full_size(layout, mode):
    # the batch-32 GQA4 workload at full size: every output checked
    case = W.decode_gqa4_batch(poison=True, layout=layout)
    note(f"decode gqa4 batch32 full {layout}")
    got = run_decode(case, mode=mode)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, "gqa4 batch")
    assert_lse_close(got["lse"], lse)


@pytest.mark.parametrize("mode", MODES)
def test_long_mqa_split_k_full_size(mode):
    # batch 8 x 32768 tokens, 32 q heads on 1 kv head, 16 partitions + merge
    case = W.decode_mqa_long()
    note("decode mqa long split-k full")
    got = run_decode(case, mode=mode, with_ws_view=True)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, "mqa long")
    assert_lse_close(got["lse"], lse)
    assert np.isfinite(got["lse_part"]).all()       # 16 partitions of 128 pages, all live


@pytest.mark.parametrize("mode", MODES)
def test_argmax_probe_is_bit_exact_for_every_position(mode):
    # Sequence b makes key j*_b dominate by a logit margin of thousands: the
    # output must be V[j*_b] bit for bit, which pins the page-table indexing.
    rng = np.random.default_rng(5)
    L, hkv, hq = 70, 2, 8
    B = L
    case = W.decode_case(5, batch=B, num_qo_heads=hq, num_kv_heads=hkv, seq_lens=[L] * B,
                         num_pages=B * 5 + 7)
    kv = case.kv
    q = np.zeros((B, hq, 128), np.float64)
    q[:, :, 0] = 1.0
    kpool = bf16.to_f64(kv.k_pool)
    kpool[..., 0] = -1.0
    for b in range(B):
        j = b  # probe position b in sequence b
        page = kv.page_indices[kv.page_indptr[b] + j // 16]
        kpool[page, j % 16, :, 0] = 3000.0
    kv.k_pool = bf16.from_f64(kpool)
    case.q = bf16.from_f64(q)
    note("decode argmax probe")
    got = run_decode(case, mode=mode)
    for b in range(B):
        page = kv.page_indices[kv.page_indptr[b] + b // 16]
        want = np.repeat(kv.v_pool[page, b % 16], hq // hkv, axis=0)
        assert np.array_equal(got["o"][b], want), b


@pytest.mark.parametrize("mode", MODES)
def test_page_reuse_and_determinism(mode):
    case = W.decode_case(9, batch=2, num_qo_heads=8, num_kv_heads=2, seq_lens=[300, 300])
    kv = case.kv
    n = int(kv.page_indptr[1])
    kv.page_indices[n:] = kv.page_indices[:n]     # both sequences read the same pages
    case.q[1] = case.q[0]
    note("decode page reuse")
    g1 = run_decode(case, mode=mode)
    g2 = run_decode(case, mode=mode, num_partitions=1)
    o, lse = oracle_decode(case)
    assert_attention_close(g1["o"], o, "shared pages")
    # identical query rows over the same pages give identical bits
    assert np.array_equal(g1["o"][0], g1["o"][1])
    # the same call twice gives the same bits
    assert np.array_equal(g1["o"], g2["o"]) and np.array_equal(g1["lse"], g2["lse"])


@pytest.mark.parametrize("mode", MODES)
def test_physical_page_order_is_invisible(mode):
    # Permute the pool's pages and remap the table: the work decomposition
    # depends on lengths only, so the outputs keep every bit.
    case = W.decode_case(13, batch=6, num_qo_heads=16, num_kv_heads=4,
                         seq_lens=[5, 100, 333, 1024, 17, 700])
    note("decode page order")
    g1 = run_decode(case, mode=mode)
    kv = case.kv
    perm = np.random.default_rng(3).permutation(kv.num_pages)
    inv = np.argsort(perm)
    kv.k_pool = np.ascontiguousarray(kv.k_pool[perm])
    kv.v_pool = np.ascontiguousarray(kv.v_pool[perm])
    kv.page_indices = inv[kv.page_indices].astype(np.int32)
    g2 = run_decode(case, mode=mode)
    assert np.array_equal(g1["o"], g2["o"]) and np.array_equal(g1["lse"], g2["lse"])


@pytest.mark.parametrize("P", [1, 4])
@pytest.mark.parametrize("mode", MODES)
def test_one_long_sequence(P, mode):
    # 20,000 tokens on one kv head, four q heads: with P = 4 the partitions
    # hold 313 pages each, the last one a ragged 312.
    case = W.decode_case(17, batch=1, num_qo_heads=4, num_kv_heads=1, seq_lens=[20000],
                         num_partitions=P, poison=True)
    note(f"decode one long sequence P={P}")
    got = run_decode(case, mode=mode, with_ws_view=True)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"long single P={P}")
    assert_lse_close(got["lse"], lse)
    # a second call with other lengths, through the same code path
    case2 = W.decode_case(18, batch=3, num_qo_heads=4, num_kv_heads=1,
                          seq_lens=[9000, 33, 4000], num_partitions=P, poison=True)
    got2 = run_decode(case2, mode=mode)
    o2, lse2 = oracle_decode(case2)
    assert (got2["status"] == 0).all()
    assert_attention_close(got2["o"], o2, f"second call P={P}")


@pytest.mark.parametrize("mode", MODES)
def test_batch_of_300_short_sequences(mode):
    # 300 short sequences of mixed lengths
    lens = [int(x) for x in np.random.default_rng(21).integers(1, 300, size=300)]
    case = W.decode_case(21, batch=300, num_qo_heads=8, num_kv_heads=2, seq_lens=lens,
                         poison=True)
    note("decode batch 300")
    got = run_decode(case, mode=mode)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, "batch 300")
    assert_lse_close(got["lse"], lse)


@pytest.mark.parametrize("mode", MODES)
def test_device_status_flags_bad_sequences_only(mode):
    lens = [40, 40, 40, 40]
    case = W.decode_case(11, batch=4, num_qo_heads=8, num_kv_heads=2, seq_lens=lens,
                         num_pages=20)
    kv = case.kv
    kv.page_indices[kv.page_indptr[1] + 2] = 20          # seq 1: page id outside the pool
    kv.seq_lens[2] = 0                                   # seq 2: empty
    kv.seq_lens[3] = 49                                  # seq 3: needs 4 pages, lists 3
    note("decode status")
    got = run_decode(case, mode=mode, max_seq_len=64)
    assert got["status"].tolist() == [0, oxa.OXA_DEV_PAGE_RANGE, oxa.OXA_DEV_SEQ_LEN,
                                      oxa.OXA_DEV_INDPTR]
    reasons = A.decode_status(kv.seq_lens, kv.page_indptr, len(kv.page_indices),
                              kv.page_indices, kv.num_pages, 64)
    assert reasons == [None, "page_range", "seq_len", "indptr"]
    o, _ = A.paged_decode(case.q[:1], kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                          kv.page_indices, kv.seq_lens, case.sm_scale)
    assert_attention_close(got["o"][:1], o, "valid sequence next to bad ones")
    # length above the declared maximum
    got = run_decode(case, mode=mode, max_seq_len=39)
    assert got["status"][0] == oxa.OXA_DEV_SEQ_LEN


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("P", [1, 3])
@pytest.mark.parametrize("mode", MODES)
def test_batch_64_mixed_lengths(layout, P, mode):
    # 64 sequences of 1 to 3000 tokens: every output is checked, and with
    # P > 1 every partition state in the workspace.
    lens = [int(x) for x in np.random.default_rng(31).integers(1, 3000, size=64)]
    lens[5] = 1
    lens[9] = 3000
    case = W.decode_case(31 + P, batch=64, num_qo_heads=8, num_kv_heads=2, seq_lens=lens,
                         num_partitions=P, layout=layout, poison=True)
    note(f"decode batch 64 mixed {layout} P={P}")
    got = run_decode(case, mode=mode, with_ws_view=True)
    o, lse = oracle_decode(case)
    assert (got["status"] == 0).all()
    assert_attention_close(got["o"], o, f"batch 64 {layout} P={P}")
    assert_lse_close(got["lse"], lse)
    if P > 1:
        kv = case.kv
        op, lp = A.decode_partials(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                   kv.page_indices, kv.seq_lens, case.sm_scale, P,
                                   case.max_seq_len)
        live = np.isfinite(lp)
        assert np.array_equal(np.isfinite(got["lse_part"]), live)
        np.testing.assert_allclose(got["lse_part"][live], lp[live], rtol=1e-4, atol=2e-4)
        assert not got["o_part"][~live].any()
        err = got["o_part"][live] - op[live]
        assert np.max(np.abs(err)) <= 2e-2
        assert np.linalg.norm(err) / np.linalg.norm(op[live]) <= 5e-3


@pytest.mark.parametrize("mode", MODES)
def test_bad_sequences_among_80(mode):
    # Invalid sequences among 80: each bad one is flagged, and the valid ones
    # around them still come out right.
    lens = [int(x) for x in np.random.default_rng(41).integers(500, 2500, size=80)]
    case = W.decode_case(41, batch=80, num_qo_heads=8, num_kv_heads=2, seq_lens=lens,
                         poison=True)
    kv = case.kv
    kv.seq_lens[3] = 0                                    # empty
    kv.page_indices[kv.page_indptr[7] + 1] = kv.num_pages  # a page id outside the pool
    kv.seq_lens[11] = int(kv.page_indptr[12] - kv.page_indptr[11]) * 16 + 1  # too few pages
    msl = int(kv.seq_lens.max())
    note("decode bad sequences among 80")
    got = run_decode(case, mode=mode, max_seq_len=msl)
    want = [0] * 80
    want[3], want[7], want[11] = oxa.OXA_DEV_SEQ_LEN, oxa.OXA_DEV_PAGE_RANGE, oxa.OXA_DEV_INDPTR
    assert got["status"].tolist() == want
    good = [b for b in range(80) if want[b] == 0]
    indptr, idx = [0], []
    for b in good:
        idx.extend(kv.page_indices[kv.page_indptr[b]:kv.page_indptr[b + 1]])
        indptr.append(len(idx))
    o, _ = A.paged_decode(case.q[good], kv.k_pool, kv.v_pool, kv.layout,
                          np.array(indptr, np.int32), np.array(idx, np.int32),
                          kv.seq_lens[good], case.sm_scale)
    assert_attention_close(got["o"][good], o, "valid sequences among bad ones")
