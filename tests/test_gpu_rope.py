"""Standalone NeoX RoPE on the GPU vs the FP64 oracle, bit for bit.

Both sides give the double-precision rotation of the bf16 inputs rounded once
to bf16 (the kernel forms it in f32 where that provably rounds the same and in
double otherwise), so the outputs must agree exactly: q and k together and
each alone, in place, over positions 0 .. 32767, negative and extreme int32
positions, the Llama 3.1 frequency table, pairs built to cancel (which send
many outputs down the double-precision path), and the 32768-token
long-prefill shape.  The standalone op must also give the same bits as the
fused RoPE + append.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import bf16 as B
from oracle import rope as R
from tests.gpu_helpers import dev, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu

D = 128
LLAMA31 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192)


def _inputs(seed, nnz, hq, hkv, lo=0, hi=32767):
    rng = np.random.default_rng(seed)
    q = W.bf16_normal(rng, (nnz, hq, D))
    k = W.bf16_normal(rng, (nnz, hkv, D))
    pos = rng.integers(lo, hi, size=nnz, endpoint=True).astype(np.int32)
    return q, k, pos


@pytest.mark.parametrize("sides", ["qk", "q", "k"])
def test_rope_neox_bit_exact(sides):
    nnz, hq, hkv = 777, 32, 8
    q, k, pos = _inputs(4000, nnz, hq, hkv)
    pos[:2] = [0, 32767]
    ensure_built()
    qi = dev(q) if "q" in sides else None
    ki = dev(k) if "k" in sides else None
    qo = torch.empty_like(qi) if qi is not None else None
    ko = torch.empty_like(ki) if ki is not None else None
    note(f"rope_neox {sides} nnz={nnz}")
    assert oxa.oxa_rope_neox(qi, qo, ki, ko, dev(pos), rope_theta=10000.0) == oxa.OXA_OK
    torch.cuda.synchronize()
    if qo is not None:
        assert np.array_equal(host_bits(qo), R.rope_neox_bf16(q, pos, 10000.0))
    if ko is not None:
        assert np.array_equal(host_bits(ko), R.rope_neox_bf16(k, pos, 10000.0))


def test_rope_cancelling_pairs_bit_exact():
    """x2 = bf16(x1 cot(angle)) for every pair, so x1 cos - x2 sin nearly
    cancels: the rotated value is a small fraction of |x1| + |x2|, and many
    outputs lie within the f32 form's error bound of a bf16 rounding
    boundary (or below the size it needs), taking the double-precision path."""
    nnz, hq, hkv = 256, 8, 2
    rng = np.random.default_rng(4010)
    pos = rng.integers(1, 32767, size=nnz, endpoint=True).astype(np.int32)
    angle = pos[:, None].astype(np.float64) * R.inv_freq(10000.0, D)[None, :]   # [nnz, 64]
    cot = np.cos(angle) / np.sin(angle)

    def pairs(h):
        x1 = B.to_f64(W.bf16_normal(rng, (nnz, h, D // 2)))
        return B.from_f64(np.concatenate([x1, x1 * cot[:, None, :]], axis=-1))

    q, k = pairs(hq), pairs(hkv)
    # the inputs do cancel: the first half of the rotation is small against the inputs
    x = B.to_f64(q)
    y = R.rope_neox(x, pos[:, None], 10000.0)
    ratio = np.abs(y[..., :D // 2]) / (np.abs(x[..., :D // 2]) + np.abs(x[..., D // 2:]))
    assert np.median(ratio) < 2.0 ** -6
    ensure_built()
    qi, ki = dev(q), dev(k)
    qo, ko = torch.empty_like(qi), torch.empty_like(ki)
    note("rope_neox cancelling pairs")
    assert oxa.oxa_rope_neox(qi, qo, ki, ko, dev(pos), rope_theta=10000.0) == oxa.OXA_OK
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qo), R.rope_neox_bf16(q, pos, 10000.0))
    assert np.array_equal(host_bits(ko), R.rope_neox_bf16(k, pos, 10000.0))


def test_rope_in_place_equals_out_of_place():
    q, k, pos = _inputs(4001, 300, 16, 4)
    ensure_built()
    qi, ki, p = dev(q), dev(k), dev(pos)
    qo, ko = torch.empty_like(qi), torch.empty_like(ki)
    note("rope_neox in place")
    assert oxa.oxa_rope_neox(qi, qo, ki, ko, p) == oxa.OXA_OK
    assert oxa.oxa_rope_neox(qi, qi, ki, ki, p) == oxa.OXA_OK
    torch.cuda.synchronize()
    assert torch.equal(qi, qo) and torch.equal(ki, ko)


def test_rope_extreme_and_negative_positions():
    nnz = 64
    q, k, _ = _inputs(4002, nnz, 8, 2)
    rng = np.random.default_rng(4003)
    pos = np.concatenate([
        np.array([-1, -32768, 2**31 - 1, -2**31, 1_000_000, -1_000_003, 65536, 131071],
                 dtype=np.int64),
        rng.integers(-2**31, 2**31 - 1, size=nnz - 8)]).astype(np.int32)
    ensure_built()
    qo, ko = torch.empty(q.shape, dtype=torch.int16, device="cuda"), \
        torch.empty(k.shape, dtype=torch.int16, device="cuda")
    note("rope_neox extreme positions")
    assert oxa.oxa_rope_neox(dev(q), qo, dev(k), ko, dev(pos)) == oxa.OXA_OK
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qo), R.rope_neox_bf16(q, pos, 10000.0))
    assert np.array_equal(host_bits(ko), R.rope_neox_bf16(k, pos, 10000.0))


def test_rope_llama31_bit_exact():
    nnz, hq, hkv = 513, 32, 8
    q, k, pos = _inputs(4004, nnz, hq, hkv, 0, 131071)
    ensure_built()
    qo, ko = torch.empty(q.shape, dtype=torch.int16, device="cuda"), \
        torch.empty(k.shape, dtype=torch.int16, device="cuda")
    note("rope_llama31")
    assert oxa.oxa_rope_llama31(dev(q), qo, dev(k), ko, dev(pos), rope_theta=500000.0,
                                **LLAMA31) == oxa.OXA_OK
    torch.cuda.synchronize()
    table = R.inv_freq_llama31(500000.0, D, **LLAMA31)
    assert np.array_equal(host_bits(qo), R.rope_neox_bf16(q, pos, None, table))
    assert np.array_equal(host_bits(ko), R.rope_neox_bf16(k, pos, None, table))
    # the rescaled table really differs from the standard one on these inputs
    assert not np.array_equal(host_bits(ko), R.rope_neox_bf16(k, pos, 500000.0))


def test_rope_long_prefill_shape_and_fused_append_agree():
    """32768 tokens (2 x 16384, positions 0..16383 twice), 32 q / 8 kv heads:
    every k bit against the oracle, q on 2048 sampled tokens, and all of q and
    k against what the fused RoPE + append wrote (q_out, and k in the pages)."""
    case = W.rope_append_prefill()
    kv = case.kv
    nnz = case.k.shape[0]
    ensure_built()
    qi, ki, p = dev(case.q), dev(case.k), dev(case.positions)
    qo, ko = torch.empty_like(qi), torch.empty_like(ki)
    note("rope_neox 32768 tokens")
    assert oxa.oxa_rope_neox(qi, qo, ki, ko, p, rope_theta=case.rope_theta) == oxa.OXA_OK
    torch.cuda.synchronize()
    k_bits = host_bits(ko)
    assert np.array_equal(k_bits, R.rope_neox_bf16(case.k, case.positions, case.rope_theta))
    sample = np.random.default_rng(4005).choice(nnz, 2048, replace=False)
    assert np.array_equal(host_bits(qo)[sample],
                          R.rope_neox_bf16(case.q[sample], case.positions[sample],
                                           case.rope_theta))
    # the fused op on the same tokens
    kp, vp = dev(kv.k_pool), dev(kv.v_pool)
    q_rot = torch.empty_like(qi)
    status = torch.full((2,), 9, dtype=torch.int32, device="cuda")
    note("fused append on the same 32768 tokens")
    rc = oxa.oxa_paged_append_rope(qi, q_rot, ki, dev(case.v), dev(case.batch_indices), p, kp, vp,
                                   dev(kv.page_indptr), dev(kv.page_indices),
                                   dev(case.page_refcounts), status, layout=kv.layout,
                                   rope_theta=case.rope_theta)
    assert rc == oxa.OXA_OK
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, -1]
    assert torch.equal(q_rot, qo)
    # k rows as the pages hold them, in token order
    pages = kv.page_indices[kv.page_indptr[case.batch_indices] + case.positions // 16]
    slots = case.positions % 16
    kp_bits = host_bits(kp)
    assert np.array_equal(kp_bits[pages, slots], k_bits)
