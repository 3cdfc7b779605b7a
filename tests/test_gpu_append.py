"""Fused RoPE + paged append on the GPU vs the FP64 oracle (bit-exact indexing)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rope as R
from tests.gpu_helpers import dev, host, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu

REASON = {None: 0, "page_range": oxa.OXA_DEV_PAGE_RANGE, "not_exclusive": oxa.OXA_DEV_NOT_EXCLUSIVE,
          "capacity": oxa.OXA_DEV_CAPACITY, "batch_index": oxa.OXA_DEV_BATCH_INDEX}


def run_append(case, *, with_q=True, in_place=False, batch_indices=None, positions=None,
               page_indices=None, refcounts=None):
    ensure_built()
    kv = case.kv
    bi = case.batch_indices if batch_indices is None else batch_indices
    pos = case.positions if positions is None else positions
    ids = kv.page_indices if page_indices is None else page_indices
    rc = case.page_refcounts if refcounts is None else refcounts
    q_in = dev(case.q) if with_q else None
    q_out = (q_in if in_place else torch.empty_like(q_in)) if with_q else None
    if with_q and not in_place:
        q_out.fill_(0x1234)
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    status = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    code = oxa.oxa_paged_append_rope(q_in, q_out, dev(case.k), dev(case.v), dev(bi), dev(pos), kp,
                                     vp, dev(kv.page_indptr), dev(ids), dev(rc), status,
                                     layout=kv.layout, rope_theta=case.rope_theta)
    assert code == oxa.OXA_OK, oxa.status_string(code)
    torch.cuda.synchronize()
    return dict(q_out=host_bits(q_out) if with_q else None, k=host_bits(kp), v=host_bits(vp),
                status=host(status))


def oracle_append(case, *, with_q=True, batch_indices=None, positions=None, page_indices=None,
                  refcounts=None):
    kv = case.kv
    return R.paged_append_rope(
        case.q if with_q else None, case.k, case.v,
        case.batch_indices if batch_indices is None else batch_indices,
        case.positions if positions is None else positions, kv.k_pool, kv.v_pool, kv.layout,
        kv.page_indptr, kv.page_indices if page_indices is None else page_indices,
        case.page_refcounts if refcounts is None else refcounts, case.rope_theta)


def ulp_diff(a, b):
    """Distance in bf16 units in the last place (same-sign finite values)."""
    ia = a.astype(np.int32)
    ib = b.astype(np.int32)
    ia = np.where(ia & 0x8000, 0x8000 - ia, ia)
    ib = np.where(ib & 0x8000, 0x8000 - ib, ib)
    return np.abs(ia - ib)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("in_place", [False, True])
def test_append_matches_oracle(layout, in_place):
    case = W.append_case(21, seq_lens=[5, 37, 16, 64], num_qo_heads=8, num_kv_heads=2,
                         layout=layout, extra_pages=1, spare_pages=5)
    note(f"append {layout} in_place={in_place}")
    got = run_append(case, in_place=in_place)
    reason, q_ref, k_ref, v_ref = oracle_append(case)
    assert reason is None and got["status"].tolist() == [0, -1]
    assert np.array_equal(got["v"], v_ref)                   # V bytes: exact copy into slots
    assert np.array_equal(got["k"], k_ref)                   # rotated K + untouched sentinels
    assert np.array_equal(got["q_out"], q_ref)


def test_append_without_q_and_high_positions():
    # positions up to 32767 (2048 pages listed for one sequence): RoPE at large
    # angles and page indexing at the far end of a long page list
    rng = np.random.default_rng(3)
    case = W.append_case(22, seq_lens=[32768], num_qo_heads=4, num_kv_heads=2,
                         spare_pages=4)
    keep = np.concatenate([np.arange(0, 40), np.arange(16000, 16040), np.arange(32700, 32768)])
    case.q, case.k, case.v = case.q[keep], case.k[keep], case.v[keep]
    case.batch_indices, case.positions = case.batch_indices[keep], case.positions[keep]
    note("append high positions")
    got = run_append(case)
    reason, q_ref, k_ref, v_ref = oracle_append(case)
    assert reason is None and got["status"][0] == 0
    assert np.array_equal(got["v"], v_ref)
    d = ulp_diff(got["q_out"], q_ref)
    assert d.max() <= 1 and np.count_nonzero(d) == 0, f"{np.count_nonzero(d)} q values differ"
    assert np.array_equal(got["k"], k_ref)
    got2 = run_append(case, with_q=False)
    assert np.array_equal(got2["k"], k_ref) and np.array_equal(got2["v"], v_ref)


def test_rejections_write_nothing():
    case = W.append_case(23, seq_lens=[20, 9, 33], num_qo_heads=4, num_kv_heads=1)
    kv = case.kv
    checks = []
    rc = case.page_refcounts.copy()
    rc[kv.page_indices[1]] = 2
    checks.append(dict(refcounts=rc))
    pos = case.positions.copy()
    pos[25] = 16                                   # sequence 1 lists 1 page = 16 slots
    checks.append(dict(positions=pos))
    ids = kv.page_indices.copy()
    ids[3] = kv.num_pages + 5
    checks.append(dict(page_indices=ids))
    bi = case.batch_indices.copy()
    bi[40] = 3
    bi[50] = -1
    checks.append(dict(batch_indices=bi))
    for over in checks:
        reason, _, k_ref, v_ref = oracle_append(case, **over)
        bad = R.append_status(over.get("batch_indices", case.batch_indices),
                              over.get("positions", case.positions), kv.page_indptr,
                              over.get("page_indices", kv.page_indices),
                              over.get("refcounts", case.page_refcounts), kv.num_pages, 3)
        note(f"append rejection {reason}")
        got = run_append(case, **over)
        assert got["status"].tolist() == [REASON[reason], bad[0]]
        assert np.array_equal(got["k"], kv.k_pool) and np.array_equal(got["v"], kv.v_pool)
        assert (got["q_out"] == 0x1234).all()      # q_out untouched too


def test_rejection_spread_over_check_groups():
    # 5000 tokens: the check pass runs five work-groups of 1024 tokens each;
    # the lowest failing token must win whichever group saw it, and a failure
    # seen only by the last group must still stop every write.
    case = W.append_case(29, seq_lens=[3000, 2000], num_qo_heads=4, num_kv_heads=2)
    kv = case.kv
    pos = case.positions.copy()
    pos[4500] = 10 ** 6                            # far beyond sequence 1's pages
    bi = case.batch_indices.copy()
    bi[2100] = 7                                   # a sequence that does not exist
    rc = case.page_refcounts.copy()
    rc[kv.page_indices[kv.page_indptr[1] + 124]] = 0   # the page of token 3000 + 1984
    for over in (dict(positions=pos), dict(batch_indices=bi), dict(refcounts=rc),
                 dict(positions=pos, batch_indices=bi, refcounts=rc)):
        reason, _, _, _ = oracle_append(case, **over)
        bad = R.append_status(over.get("batch_indices", case.batch_indices),
                              over.get("positions", case.positions), kv.page_indptr,
                              kv.page_indices, over.get("refcounts", case.page_refcounts),
                              kv.num_pages, 2)
        note(f"append spread rejection {sorted(over)}")
        got = run_append(case, **over)
        assert got["status"].tolist() == [REASON[reason], bad[0]]
        assert np.array_equal(got["k"], kv.k_pool) and np.array_equal(got["v"], kv.v_pool)
        assert (got["q_out"] == 0x1234).all()


def test_empty_append_reports_success():
    case = W.append_case(31, seq_lens=[0, 0], num_qo_heads=4, num_kv_heads=1, extra_pages=1)
    note("append nnz=0")
    got = run_append(case)
    assert got["status"].tolist() == [0, -1]
    assert np.array_equal(got["k"], case.kv.k_pool) and np.array_equal(got["v"], case.kv.v_pool)


def test_rope_append_full_size():
    # 2 x 16384 tokens, 32 q / 8 kv heads, positions 0..16383, 2048 exclusive pages
    case = W.rope_append_prefill()
    note("append full size")
    got = run_append(case)
    reason, q_ref, k_ref, v_ref = oracle_append(case)
    assert reason is None and got["status"].tolist() == [0, -1]
    assert np.array_equal(got["v"], v_ref)
    assert np.array_equal(got["k"], k_ref)
    d = ulp_diff(got["q_out"], q_ref)
    assert d.max() <= 1, "q differs by more than one bf16 ulp"
    assert np.count_nonzero(d) == 0, f"{np.count_nonzero(d)} q values differ by 1 ulp"


def run_plain(case, *, refcounts=None, positions=None, kp=None, vp=None):
    ensure_built()
    kv = case.kv
    kp = dev(kv.k_pool) if kp is None else kp
    vp = dev(kv.v_pool) if vp is None else vp
    status = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    code = oxa.oxa_paged_append(dev(case.k), dev(case.v), dev(case.batch_indices),
                                dev(case.positions if positions is None else positions), kp, vp,
                                dev(kv.page_indptr), dev(kv.page_indices),
                                dev(case.page_refcounts if refcounts is None else refcounts),
                                status, layout=kv.layout)
    assert code == oxa.OXA_OK, oxa.status_string(code)
    torch.cuda.synchronize()
    return host_bits(kp), host_bits(vp), host(status)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_plain_append_matches_oracle(layout):
    case = W.append_case(31, seq_lens=[5, 37, 16, 64, 1], num_qo_heads=8, num_kv_heads=4,
                         layout=layout, extra_pages=1, spare_pages=5)
    note(f"plain append {layout}")
    k, v, status = run_plain(case)
    kv = case.kv
    reason, k_ref, v_ref = R.paged_append(case.k, case.v, case.batch_indices, case.positions,
                                          kv.k_pool, kv.v_pool, layout, kv.page_indptr,
                                          kv.page_indices, case.page_refcounts)
    assert reason is None and status.tolist() == [0, -1]
    assert np.array_equal(k, k_ref) and np.array_equal(v, v_ref)


def test_plain_append_rejection_writes_nothing():
    case = W.append_case(32, seq_lens=[20, 9, 33], num_qo_heads=4, num_kv_heads=2)
    kv = case.kv
    rc = case.page_refcounts.copy()
    rc[kv.page_indices[kv.page_indptr[1]]] = 2      # sequence 1's only page is shared
    note("plain append with a shared page")
    k, v, status = run_plain(case, refcounts=rc)
    reason, _, _ = R.paged_append(case.k, case.v, case.batch_indices, case.positions, kv.k_pool,
                                  kv.v_pool, kv.layout, kv.page_indptr, kv.page_indices, rc)
    first_bad = 20                                   # sequence 1's first token
    assert R.append_status(case.batch_indices, case.positions, kv.page_indptr, kv.page_indices,
                           rc, kv.num_pages, 3) == (first_bad, "not_exclusive")
    assert reason == "not_exclusive"
    assert status.tolist() == [oxa.OXA_DEV_NOT_EXCLUSIVE, first_bad]
    assert np.array_equal(k, kv.k_pool) and np.array_equal(v, kv.v_pool)


def test_plain_append_full_size_and_equal_to_fused_at_position_zero():
    """The 2 x 16384-token, 8 kv head append shape, every pool bit against the
    oracle; then one token per sequence at position 0, where the fused RoPE
    append (angle 0) must store the same bits as the plain one."""
    case = W.rope_append_prefill()
    kv = case.kv
    note("plain append 32768 tokens")
    k, v, status = run_plain(case)
    reason, k_ref, v_ref = R.paged_append(case.k, case.v, case.batch_indices, case.positions,
                                          kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                          kv.page_indices, case.page_refcounts)
    assert reason is None and status.tolist() == [0, -1]
    assert np.array_equal(k, k_ref) and np.array_equal(v, v_ref)
    small = W.append_case(33, seq_lens=[1] * 7, num_qo_heads=4, num_kv_heads=8)
    assert not small.positions.any()
    note("plain and fused append at position 0")
    k1, v1, s1 = run_plain(small)
    got = run_append(small, with_q=False)
    assert s1.tolist() == [0, -1] and got["status"].tolist() == [0, -1]
    assert np.array_equal(k1, got["k"]) and np.array_equal(v1, got["v"])
