"""Pins of the RoPE / paged-append oracle against facts outside the oracle.

* transformers' NeoX-style ``apply_rotary_pos_emb`` (rotate_half) as a library
  reference for the split-half convention;
* complex multiplication by exp(i * angle) (numpy complex) for every pair;
* closed forms of the frequency table; rotation by zero is the identity;
* the Llama 3.1 table against transformers' own llama3 rope initialisation
  (float32 there), its three bands against closed forms;
* group laws: pair norms preserved, R_p R_q = R_{p+q}, scores depend only on
  the position difference;
* append round trips through the (separately pinned) page-table gather, and
  rejection leaves the pools untouched.
"""
import numpy as np
import pytest
import torch
from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

import workloads as W
from oracle import attention as A
from oracle import bf16
from oracle import rope as R

D = 128


def test_inv_freq_closed_forms():
    f = R.inv_freq(10000.0, D)
    assert f.shape == (64,)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[32], 0.01, rtol=1e-15)          # 10000 ** (-1/2)
    np.testing.assert_allclose(f[1:] / f[:-1], 10000.0 ** (-2.0 / D), rtol=1e-14)


LLAMA31 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
               original_max_position=8192)


def test_llama31_table_matches_transformers():
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    cfg = LlamaConfig(hidden_size=32 * D, num_attention_heads=32, head_dim=D,
                      max_position_embeddings=131072,
                      rope_parameters={"rope_type": "llama3", "rope_theta": 500000.0,
                                       "factor": 8.0, "low_freq_factor": 1.0,
                                       "high_freq_factor": 4.0,
                                       "original_max_position_embeddings": 8192})
    ref, _ = ROPE_INIT_FUNCTIONS["llama3"](cfg, "cpu")
    got = R.inv_freq_llama31(500000.0, D, **LLAMA31)
    np.testing.assert_allclose(got, ref.double().numpy(), rtol=2e-6)


def test_llama31_bands():
    base = R.inv_freq(500000.0, D)
    got = R.inv_freq_llama31(500000.0, D, **LLAMA31)
    wl = 2 * np.pi / base
    hi = wl < 8192 / 4.0
    lo = wl > 8192 / 1.0
    assert hi.any() and lo.any() and (~hi & ~lo).any()
    assert np.array_equal(got[hi], base[hi])          # short wavelengths keep their frequency
    assert np.array_equal(got[lo], base[lo] / 8.0)    # long ones are slowed by the factor
    mid = ~hi & ~lo                                   # in between: strictly between the two
    assert (got[mid] < base[mid]).all() and (got[mid] > base[mid] / 8.0).all()
    # with factor 1 the table is the standard one
    same = R.inv_freq_llama31(500000.0, D, 1.0, 1.0, 4.0, 8192)
    np.testing.assert_allclose(same, base, rtol=1e-15)


def test_rope_with_a_table_and_negative_positions():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, D))
    pos = rng.integers(-40000, 40000, size=20)
    table = R.inv_freq_llama31(500000.0, D, **LLAMA31)
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * pos[:, None] * table)
    got = R.rope_neox(x, pos, None, freqs=table)
    np.testing.assert_allclose(got[:, :64], z.real, atol=1e-12)
    np.testing.assert_allclose(got[:, 64:], z.imag, atol=1e-12)
    # rotating by p then by -p returns the input
    back = R.rope_neox(R.rope_neox(x, pos, 10000.0), -pos, 10000.0)
    np.testing.assert_allclose(back, x, atol=1e-12)


def test_matches_transformers_rotate_half():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, D))
    pos = rng.integers(0, 32768, size=50)
    inv = torch.from_numpy(R.inv_freq(10000.0, D))
    freqs = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None, :]
    emb = torch.cat([freqs, freqs], dim=-1)
    xt = torch.from_numpy(x)
    ref, _ = apply_rotary_pos_emb(xt, xt, emb.cos(), emb.sin(), unsqueeze_dim=1)
    got = R.rope_neox(x, pos[:, None], 10000.0)
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


def test_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, D))
    pos = rng.integers(0, 32768, size=40)
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * pos[:, None] * R.inv_freq(10000.0, D))
    got = R.rope_neox(x, pos, 10000.0)
    np.testing.assert_allclose(got[:, :64], z.real, atol=1e-13)
    np.testing.assert_allclose(got[:, 64:], z.imag, atol=1e-13)


def test_position_zero_is_identity_bit_exact():
    rng = np.random.default_rng(2)
    xb = W.bf16_normal(rng, (30, 4, D))
    out = R.rope_neox_bf16(xb, np.zeros(30, np.int32), 10000.0)
    assert np.array_equal(out, xb)


def test_group_laws():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, D))
    y = rng.standard_normal((20, D))
    p = rng.integers(0, 16384, size=20)
    q = rng.integers(0, 16384, size=20)
    rx = R.rope_neox(x, p, 10000.0)
    # pair norms are preserved
    np.testing.assert_allclose(rx[:, :64] ** 2 + rx[:, 64:] ** 2, x[:, :64] ** 2 + x[:, 64:] ** 2,
                               rtol=1e-12)
    # composition: rotating by q after p equals rotating by p + q
    np.testing.assert_allclose(R.rope_neox(rx, q, 10000.0), R.rope_neox(x, p + q, 10000.0),
                               atol=1e-10)
    # scores depend only on the position difference
    s1 = np.einsum("nd,nd->n", R.rope_neox(x, p + 7, 10000.0), R.rope_neox(y, q + 7, 10000.0))
    s2 = np.einsum("nd,nd->n", R.rope_neox(x, p + 5000, 10000.0), R.rope_neox(y, q + 5000, 10000.0))
    np.testing.assert_allclose(s1, s2, atol=1e-10)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_append_round_trip_and_untouched_slots(layout):
    case = W.append_case(5, seq_lens=[5, 37, 16], num_qo_heads=8, num_kv_heads=2, layout=layout,
                         extra_pages=1, spare_pages=3)
    kv = case.kv
    reason, q_out, kp, vp = R.paged_append_rope(
        case.q, case.k, case.v, case.batch_indices, case.positions, kv.k_pool, kv.v_pool, layout,
        kv.page_indptr, kv.page_indices, case.page_refcounts, case.rope_theta)
    assert reason is None
    k_rot = R.rope_neox_bf16(case.k, case.positions, case.rope_theta)
    assert np.array_equal(q_out, R.rope_neox_bf16(case.q, case.positions, case.rope_theta))
    written = np.zeros(kp.shape, dtype=bool)
    for b, n in enumerate([5, 37, 16]):
        s = int(case.qo_indptr[b])
        # gather is pinned on its own (hand-derived fixture); use it to read back
        kb = A.gather(kp, layout, kv.page_indptr, kv.page_indices, b, n)
        vb = A.gather(vp, layout, kv.page_indptr, kv.page_indices, b, n)
        assert np.array_equal(kb, bf16.to_f64(k_rot[s:s + n]))
        assert np.array_equal(vb, bf16.to_f64(case.v[s:s + n]))
    # count untouched slots: everything except the written (page, slot) rows
    n_tokens = 5 + 37 + 16
    assert np.count_nonzero(kp != 0x5A5A) <= n_tokens * 2 * D
    assert np.count_nonzero(vp == 0xA5A5) == vp.size - n_tokens * 2 * D + np.count_nonzero(
        case.v == 0xA5A5)


def _reject(case, **over):
    kv = case.kv
    args = dict(batch_indices=case.batch_indices.copy(), positions=case.positions.copy(),
                page_indices=kv.page_indices.copy(), page_refcounts=case.page_refcounts.copy())
    args.update(over)
    return R.paged_append_rope(case.q, case.k, case.v, args["batch_indices"], args["positions"],
                               kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                               args["page_indices"], args["page_refcounts"], case.rope_theta)


def test_append_rejections_write_nothing():
    case = W.append_case(6, seq_lens=[20, 9], num_qo_heads=4, num_kv_heads=1)
    kv = case.kv
    rc = case.page_refcounts.copy()
    rc[kv.page_indices[1]] = 2                      # second page of sequence 0 is shared
    reason, q_out, kp, vp = _reject(case, page_refcounts=rc)
    assert reason == "not_exclusive" and q_out is None
    assert np.array_equal(kp, kv.k_pool) and np.array_equal(vp, kv.v_pool)
    pos = case.positions.copy()
    pos[3] = 32                                     # sequence 0 owns 2 pages = 32 slots
    assert _reject(case, positions=pos)[0] == "capacity"
    pos[3] = -1
    assert _reject(case, positions=pos)[0] == "capacity"
    ids = kv.page_indices.copy()
    ids[2] = kv.num_pages                           # first page of sequence 1 out of the pool
    assert _reject(case, page_indices=ids)[0] == "page_range"
    bi = case.batch_indices.copy()
    bi[-1] = 2
    assert _reject(case, batch_indices=bi)[0] == "batch_index"
    # the first failing token decides the reason
    bi[0] = -1
    assert R.append_status(bi, pos, kv.page_indptr, ids, case.page_refcounts, kv.num_pages,
                           2) == (0, "batch_index")
    rc0 = np.zeros_like(case.page_refcounts)
    assert _reject(case, page_refcounts=rc0)[0] == "not_exclusive"


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_plain_append_round_trip(layout):
    """Plain append read back through the (separately pinned) gather: every
    sequence's rows are exactly the k and v given, and no other slot moves."""
    lens = [5, 37, 16]
    case = W.append_case(7, seq_lens=lens, num_qo_heads=8, num_kv_heads=2, layout=layout,
                         extra_pages=1, spare_pages=3)
    kv = case.kv
    reason, kp, vp = R.paged_append(case.k, case.v, case.batch_indices, case.positions,
                                    kv.k_pool, kv.v_pool, layout, kv.page_indptr,
                                    kv.page_indices, case.page_refcounts)
    assert reason is None
    for b, n in enumerate(lens):
        s = int(case.qo_indptr[b])
        assert np.array_equal(A.gather(kp, layout, kv.page_indptr, kv.page_indices, b, n),
                              bf16.to_f64(case.k[s:s + n]))
        assert np.array_equal(A.gather(vp, layout, kv.page_indptr, kv.page_indices, b, n),
                              bf16.to_f64(case.v[s:s + n]))
    n_rows = sum(lens) * 2 * D                      # elements written per pool
    assert np.count_nonzero(kp != kv.k_pool) <= n_rows
    assert np.count_nonzero(vp != kv.v_pool) <= n_rows


def test_plain_append_equals_fused_append_at_position_zero():
    """At position 0 the rotation angle is 0 for every pair (cos 1, sin 0), so
    the fused RoPE append must store exactly what the plain append stores."""
    B = 6
    case = W.append_case(8, seq_lens=[1] * B, num_qo_heads=4, num_kv_heads=2)
    kv = case.kv
    assert not case.positions.any()
    r1, kp1, vp1 = R.paged_append(case.k, case.v, case.batch_indices, case.positions,
                                  kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                  kv.page_indices, case.page_refcounts)
    r2, _, kp2, vp2 = R.paged_append_rope(case.q, case.k, case.v, case.batch_indices,
                                          case.positions, kv.k_pool, kv.v_pool, kv.layout,
                                          kv.page_indptr, kv.page_indices, case.page_refcounts,
                                          10000.0)
    assert r1 is None and r2 is None
    assert np.array_equal(kp1, kp2) and np.array_equal(vp1, vp2)


def test_plain_append_rejections_write_nothing():
    case = W.append_case(9, seq_lens=[20, 9], num_qo_heads=4, num_kv_heads=1)
    kv = case.kv
    rc = case.page_refcounts.copy()
    rc[kv.page_indices[0]] = 3
    reason, kp, vp = R.paged_append(case.k, case.v, case.batch_indices, case.positions,
                                    kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                                    kv.page_indices, rc)
    assert reason == "not_exclusive"
    assert np.array_equal(kp, kv.k_pool) and np.array_equal(vp, kv.v_pool)
