"""Pins of the attention oracle against facts that do not come from the oracle.

* torch's scaled_dot_product_attention and logsumexp (float64, CPU) on the
  cases they cover (non-causal; causal with as many queries as keys);
* a hand-derived page-table fixture (tests/golden/page_table_gather.json);
* closed forms (one key returns its V row; equal logits return the mean of V
  with lse = ln L);
* invariances (physical page order, read-only page reuse, NHD vs HND, GQA vs
  replicated MHA, split-K merge vs unsplit);
* brute-force argmax probes that single out one key at a time.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import bf16
from tests.oracle_helpers import scatter_pages, sdpa, torch_lse

HERE = os.path.dirname(__file__)
D = 128
SCALE = 1.0 / math.sqrt(D)


def rand_bits(rng, shape):
    return W.bf16_normal(rng, shape)


# --------------------------------------------------------------------- gather

def test_gather_matches_hand_derived_fixture():
    fx = json.load(open(os.path.join(HERE, "golden", "page_table_gather.json")))
    n, h = fx["num_pages"], fx["num_kv_heads"]
    pool = np.zeros((n, 16, h, D), dtype=np.float64)
    for p in range(n):
        pool[p, :, :, 0] = p
        pool[p, :, :, 1] = np.arange(16)[:, None]
        pool[p, :, :, 2] = np.arange(h)[None, :]
    pool_bits = bf16.from_f64(pool)
    for layout in ("NHD", "HND"):
        pb = W.to_layout(pool_bits, layout)
        for b, length in enumerate(fx["seq_lens"]):
            rows = A.gather(pb, layout, fx["page_indptr"], fx["page_indices"], b, length)
            want = np.array(fx["expected_page_slot"][str(b)], dtype=np.float64)
            assert rows.shape == (length, h, D)
            assert np.array_equal(rows[:, :, 0], np.repeat(want[:, :1], h, axis=1))
            assert np.array_equal(rows[:, :, 1], np.repeat(want[:, 1:], h, axis=1))
            assert np.array_equal(rows[:, :, 2], np.tile(np.arange(h), (length, 1)))


# ------------------------------------------------------------------ the core

@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (8, 1)])
@pytest.mark.parametrize("L", [1, 5, 37])
def test_attend_matches_torch_sdpa(hq, hkv, L):
    rng = np.random.default_rng(L * 100 + hq + hkv)
    q = bf16.to_f64(rand_bits(rng, (3, hq, D)))
    k = bf16.to_f64(rand_bits(rng, (L, hkv, D)))
    v = bf16.to_f64(rand_bits(rng, (L, hkv, D)))
    o, lse = A.attend(q, k, v, SCALE, causal=False)
    np.testing.assert_allclose(o, sdpa(q, k, v, SCALE, False), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch_lse(q, k, SCALE), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (4, 1)])
def test_causal_equal_lengths_matches_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(7 + hq)
    L = 41
    q = bf16.to_f64(rand_bits(rng, (L, hq, D)))
    k = bf16.to_f64(rand_bits(rng, (L, hkv, D)))
    v = bf16.to_f64(rand_bits(rng, (L, hkv, D)))
    o, _ = A.attend(q, k, v, SCALE, causal=True)
    np.testing.assert_allclose(o, sdpa(q, k, v, SCALE, True), rtol=1e-12, atol=1e-13)
    # row 0 sees only key 0: it returns V[0] exactly (closed form)
    assert np.array_equal(o[0], np.repeat(v[0], hq // hkv, axis=0))


def test_causal_alignment_is_bottom_right():
    # The last qo rows of a qo=kv causal problem are the rows of the shorter
    # query block that ends at the same key: query i of a qo-row block sees keys
    # j <= i + (kv - qo).  torch (top-left, qo == kv) supplies the reference.
    rng = np.random.default_rng(11)
    L, qo, hq, hkv = 50, 13, 4, 2
    qf = bf16.to_f64(rand_bits(rng, (L, hq, D)))
    k = bf16.to_f64(rand_bits(rng, (L, hkv, D)))
    v = bf16.to_f64(rand_bits(rng, (L, hkv, D)))
    full = sdpa(qf, k, v, SCALE, True)
    o, _ = A.attend(qf[L - qo:], k, v, SCALE, causal=True)
    np.testing.assert_allclose(o, full[L - qo:], rtol=1e-12, atol=1e-13)
    # explicit row selection inside a sequence gives the same rows
    rows = np.array([0, 5, 12])
    o2, _ = A.attend(qf[L - qo:][rows], k, v, SCALE, causal=True, q_rows=rows, qo_len=qo)
    np.testing.assert_array_equal(o2, o[rows])


def test_length_one_returns_its_v_row():
    rng = np.random.default_rng(3)
    q = bf16.to_f64(rand_bits(rng, (1, 8, D)))
    k = bf16.to_f64(rand_bits(rng, (1, 2, D)))
    v = bf16.to_f64(rand_bits(rng, (1, 2, D)))
    o, lse = A.attend(q, k, v, SCALE, causal=False)
    assert np.array_equal(o[0], np.repeat(v[0], 4, axis=0))
    np.testing.assert_allclose(lse[0], SCALE * np.einsum("hd,hd->h", q[0], np.repeat(k[0], 4, 0)),
                               rtol=1e-14)


def test_uniform_logits_give_mean_of_v_and_log_length():
    rng = np.random.default_rng(4)
    L = 300
    q = np.zeros((2, 4, D))
    k = bf16.to_f64(rand_bits(rng, (L, 1, D)))
    v = bf16.to_f64(rand_bits(rng, (L, 1, D)))
    o, lse = A.attend(q, k, v, SCALE, causal=False)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, 0].mean(axis=0), o.shape), rtol=1e-13,
                               atol=1e-15)
    np.testing.assert_allclose(lse, math.log(L), rtol=1e-15)
    # scale 0 is the same closed form for any q
    q = bf16.to_f64(rand_bits(rng, (2, 4, D)))
    o, lse = A.attend(q, k, v, 0.0, causal=False)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, 0].mean(axis=0), o.shape), rtol=1e-13,
                               atol=1e-15)


# ---------------------------------------------------------------- paged decode

def _decode_setup(seed, lens, hq, hkv, layout="NHD", extra=3):
    rng = np.random.default_rng(seed)
    ks = [rand_bits(rng, (n, hkv, D)) for n in lens]
    vs = [rand_bits(rng, (n, hkv, D)) for n in lens]
    npages = sum(-(-n // 16) for n in lens) + extra
    prng = np.random.default_rng(seed + 1)
    kp, indptr, ids = scatter_pages(ks, npages, layout, prng)
    prng = np.random.default_rng(seed + 1)
    vp, indptr2, ids2 = scatter_pages(vs, npages, layout, prng)
    assert np.array_equal(ids, ids2)
    q = rand_bits(rng, (len(lens), hq, D))
    return q, ks, vs, kp, vp, indptr, ids


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (8, 1)])
def test_paged_decode_matches_sdpa_on_logical_rows(layout, hq, hkv):
    lens = [1, 16, 17, 70]
    q, ks, vs, kp, vp, indptr, ids = _decode_setup(5, lens, hq, hkv, layout)
    o, lse = A.paged_decode(q, kp, vp, layout, indptr, ids, lens, SCALE)
    for b, n in enumerate(lens):
        qb = bf16.to_f64(q[b:b + 1])
        kb, vb = bf16.to_f64(ks[b]), bf16.to_f64(vs[b])
        np.testing.assert_allclose(o[b:b + 1], sdpa(qb, kb, vb, SCALE, False), rtol=1e-12,
                                   atol=1e-13)
        np.testing.assert_allclose(lse[b:b + 1], torch_lse(qb, kb, SCALE), rtol=1e-13)
    assert np.all(np.isfinite(o))   # NaN-filled unused slots never leak in


def test_decode_invariant_to_physical_page_order_and_layout():
    lens = [33, 100]
    q, ks, vs, kp, vp, indptr, ids = _decode_setup(6, lens, 8, 2, "NHD")
    o1, l1 = A.paged_decode(q, kp, vp, "NHD", indptr, ids, lens, SCALE)
    perm = np.random.default_rng(9).permutation(kp.shape[0])      # new physical order
    inv = np.argsort(perm)
    o2, l2 = A.paged_decode(q, kp[perm], vp[perm], "NHD", indptr, inv[ids].astype(np.int32),
                            lens, SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = A.paged_decode(q, W.to_layout(kp, "HND"), W.to_layout(vp, "HND"), "HND", indptr,
                            ids, lens, SCALE)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_decode_read_only_page_reuse():
    # Two sequences list the same physical pages: identical q gives identical output.
    lens = [45]
    q, ks, vs, kp, vp, indptr, ids = _decode_setup(7, lens, 4, 4)
    indptr2 = np.array([0, indptr[1], 2 * indptr[1]], dtype=np.int32)
    ids2 = np.concatenate([ids, ids])
    q2 = np.concatenate([q, q])
    o, lse = A.paged_decode(q2, kp, vp, "NHD", indptr2, ids2, [45, 45], SCALE)
    assert np.array_equal(o[0], o[1]) and np.array_equal(lse[0], lse[1])
    # and a prefix share: the second sequence uses only the first page
    o, _ = A.paged_decode(q2, kp, vp, "NHD", indptr2, ids2, [45, 16], SCALE)
    ref = sdpa(bf16.to_f64(q[0:1]), bf16.to_f64(ks[0][:16]), bf16.to_f64(vs[0][:16]), SCALE, False)
    np.testing.assert_allclose(o[1:2], ref, rtol=1e-12, atol=1e-13)


def test_decode_argmax_probe_selects_each_key_exactly():
    # One key per probe gets a logit at least 200 above every other key, so its
    # weight is 1 to within exp(-200) and the output is that key's V row, bit for bit.
    rng = np.random.default_rng(8)
    n, hkv, hq = 37, 2, 4
    v = rand_bits(rng, (n, hkv, D))
    q = np.zeros((1, hq, D))
    q[0, :, 0] = 1.0
    for jstar in range(n):
        k = np.zeros((n, hkv, D))
        k[:, :, 0] = -1.0
        k[jstar, :, 0] = 4000.0
        kb = bf16.from_f64(k)
        kp, indptr, ids = scatter_pages([kb], 5, "NHD", np.random.default_rng(jstar))
        vp, _, _ = scatter_pages([v], 5, "NHD", np.random.default_rng(jstar))
        o, _ = A.paged_decode(bf16.from_f64(q), kp, vp, "NHD", indptr, ids, [n], SCALE)
        assert np.array_equal(o[0], np.repeat(bf16.to_f64(v[jstar]), hq // hkv, axis=0))


def test_gqa_equals_mha_with_replicated_kv_heads():
    lens = [29, 64]
    q, ks, vs, kp, vp, indptr, ids = _decode_setup(10, lens, 8, 2)
    o1, l1 = A.paged_decode(q, kp, vp, "NHD", indptr, ids, lens, SCALE)
    o2, l2 = A.paged_decode(q, np.repeat(kp, 4, axis=2), np.repeat(vp, 4, axis=2), "NHD",
                            indptr, ids, lens, SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- split-K

def test_partition_size_closed_forms():
    assert A.partition_pages(32768, 16) == 128          # the long MQA workload
    assert A.partition_pages(4096, 1) == 256
    assert A.partition_pages(17, 2) == 1                 # 2 pages over 2 partitions
    assert A.partition_pages(1, 4) == 1


@pytest.mark.parametrize("P", [1, 2, 3, 7, 16])
def test_split_partials_merge_to_unsplit(P):
    lens = [1, 31, 200, 513]
    q, ks, vs, kp, vp, indptr, ids = _decode_setup(12, lens, 8, 1)
    o, lse = A.paged_decode(q, kp, vp, "NHD", indptr, ids, lens, SCALE)
    op, lp = A.decode_partials(q, kp, vp, "NHD", indptr, ids, lens, SCALE, P, max(lens))
    assert op.shape == (4, 8, P, D) and lp.shape == (4, 8, P)
    om, lm = A.merge_states(op, lp)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lm, lse, rtol=1e-13, atol=1e-13)
    C = A.partition_pages(max(lens), P)
    for b, n in enumerate(lens):
        npages = -(-n // 16)
        for p in range(P):
            empty = p * C >= npages
            assert np.isneginf(lp[b, :, p]).all() == empty
            if empty:
                assert not op[b, :, p].any()
    if P == 1:
        assert np.array_equal(op[:, :, 0], o) and np.array_equal(lp[:, :, 0], lse)


def test_merge_is_order_independent_and_ignores_empty_states():
    rng = np.random.default_rng(13)
    op = rng.standard_normal((3, 5, 6, D))
    lp = rng.standard_normal((3, 5, 6)) * 4
    lp[:, :, 2] = -np.inf
    o, lse = A.merge_states(op, lp)
    perm = rng.permutation(6)
    o2, lse2 = A.merge_states(op[:, :, perm], lp[:, :, perm])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)
    keep = [0, 1, 3, 4, 5]
    o3, lse3 = A.merge_states(op[:, :, keep], lp[:, :, keep])
    np.testing.assert_allclose(o3, o, rtol=1e-13, atol=1e-14)
    # a single live state comes back unchanged
    lp1 = np.full((3, 5, 6), -np.inf)
    lp1[:, :, 4] = lp[:, :, 4]
    o4, lse4 = A.merge_states(op, lp1)
    np.testing.assert_allclose(o4, op[:, :, 4], rtol=1e-15)
    assert np.array_equal(lse4, lp[:, :, 4])


# ---------------------------------------------------------------- prefill

def test_ragged_prefill_matches_sdpa_per_sequence():
    rng = np.random.default_rng(14)
    lens = [1, 17, 40]
    case = W.ragged_case(14, qo_lens=lens, num_qo_heads=8, num_kv_heads=2)
    o, lse = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr, SCALE, True)
    for b in range(3):
        s, e = case.qo_indptr[b], case.qo_indptr[b + 1]
        qb, kb, vb = (bf16.to_f64(x[s:e]) for x in (case.q, case.k, case.v))
        np.testing.assert_allclose(o[s:e], sdpa(qb, kb, vb, SCALE, True), rtol=1e-12, atol=1e-13)
        assert np.array_equal(o[s], np.repeat(vb[0], 4, axis=0))
    # selecting rows computes exactly those rows
    rows = np.array([0, 18, 57])
    o2, l2 = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr, SCALE, True,
                              rows=rows)
    assert np.array_equal(o2[rows], o[rows]) and np.isnan(o2[1]).all()


def test_paged_prefill_equals_ragged_and_last_row_equals_decode():
    rng = np.random.default_rng(15)
    lens = [20, 50]
    case = W.ragged_case(15, qo_lens=lens, num_qo_heads=4, num_kv_heads=1)
    ks = [case.k[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(2)]
    vs = [case.v[case.kv_indptr[b]:case.kv_indptr[b + 1]] for b in range(2)]
    kp, indptr, ids = scatter_pages(ks, 9, "HND", np.random.default_rng(1))
    vp, _, _ = scatter_pages(vs, 9, "HND", np.random.default_rng(1))
    o_r, l_r = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr, SCALE, True)
    o_p, l_p = A.paged_prefill(case.q, case.qo_indptr, kp, vp, "HND", indptr, ids, lens, SCALE,
                               True)
    assert np.array_equal(o_r, o_p) and np.array_equal(l_r, l_p)
    last = case.qo_indptr[1:] - 1
    o_d, l_d = A.paged_decode(case.q[last], kp, vp, "HND", indptr, ids, lens, SCALE)
    # same arithmetic, different BLAS blocking: equal to rounding
    np.testing.assert_allclose(o_d, o_p[last], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l_d, l_p[last], rtol=1e-14)


def test_paged_prefill_with_fewer_queries_than_keys():
    # a chunk of the last qo rows (bottom-right causal) against all paged keys
    rng = np.random.default_rng(16)
    L, qo = 40, 9
    k = rand_bits(rng, (L, 2, D))
    v = rand_bits(rng, (L, 2, D))
    q = rand_bits(rng, (L, 8, D))
    kp, indptr, ids = scatter_pages([k], 4, "NHD", np.random.default_rng(99))
    vp, _, _ = scatter_pages([v], 4, "NHD", np.random.default_rng(99))
    full = sdpa(bf16.to_f64(q), bf16.to_f64(k), bf16.to_f64(v), SCALE, True)
    o, _ = A.paged_prefill(q[L - qo:], np.array([0, qo], np.int32), kp, vp, "NHD", indptr, ids,
                           [L], SCALE, True)
    np.testing.assert_allclose(o, full[L - qo:], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- status

def test_decode_status_reasons():
    ids = np.array([0, 1, 2, 7], np.int32)
    ind = np.array([0, 2, 2, 4], np.int32)
    # seq 0: 20 tokens over 2 pages (ok); seq 1: 5 tokens over 0 pages; seq 2: page 7 of 4
    assert A.decode_status([20, 5, 17], ind, 4, ids, 4, 100) == [None, "indptr", "page_range"]
    assert A.decode_status([0, 5, 17], ind, 4, ids, 8, 100)[0] == "seq_len"
    assert A.decode_status([33, 1, 1], ind, 4, ids, 8, 100)[0] == "indptr"
    assert A.decode_status([20, 1, 1], ind, 4, ids, 8, 19)[0] == "seq_len"
    assert A.decode_status([20], np.array([0, 5], np.int32), 4, ids, 8, 100) == ["indptr"]


def test_prefill_status_reasons():
    assert A.ragged_status([0, 4, 6], [0, 3, 9], 6, 9, 8, 8, True) == ["causal", None]
    assert A.ragged_status([0, 4, 6], [0, 3, 9], 6, 9, 8, 8, False) == [None, None]
    assert A.ragged_status([0, 4, 7], [0, 3, 9], 6, 9, 8, 8, False) == [None, "indptr"]
    assert A.ragged_status([0, 4, 6], [0, 4, 4], 6, 9, 8, 8, False) == [None, "seq_len"]
    ids = np.array([0, 1, 9], np.int32)
    assert A.paged_prefill_status([0, 3, 5], 5, [20, 16], [0, 2, 3], 3, ids, 4, 8, 64, True) \
        == [None, "page_range"]
    assert A.paged_prefill_status([0, 3, 5], 5, [40, 16], [0, 2, 3], 3, ids, 4, 8, 64, True) \
        == ["indptr", "page_range"]
