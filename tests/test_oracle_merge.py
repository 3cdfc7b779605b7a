"""Pins of the attention-state merge oracle against facts outside it.

A state (v, lse) of a query over a key set is softmax attention over that set
and the natural-log log-sum-exp of its scaled scores.  Merging the states of
disjoint key sets must give the state of their union; torch's
scaled_dot_product_attention and logsumexp (float64, CPU) compute both sides
of that without the oracle.  Closed forms: two states with equal lse merge to
their mean with lse + ln 2; empty states (lse = -inf) drop out whatever their
v holds; all-empty gives (0, -inf); one state comes back unchanged.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from tests.oracle_helpers import sdpa, torch_lse

D = 128
SCALE = 1.0 / math.sqrt(D)


def _qkv(rng, rows, heads, keys):
    q = rng.standard_normal((rows, heads, D))
    k = rng.standard_normal((keys, heads, D)) * 1.5
    v = rng.standard_normal((keys, heads, D))
    return q, k, v


def _state(q, k, v):
    return sdpa(q, k, v, SCALE, False), torch_lse(q, k, SCALE)


@pytest.mark.parametrize("cut", [1, 37, 199])
def test_pair_of_disjoint_key_sets_merges_to_their_union(cut):
    rng = np.random.default_rng(40 + cut)
    q, k, v = _qkv(rng, 6, 4, 200)
    va, la = _state(q, k[:cut], v[:cut])
    vb, lb = _state(q, k[cut:], v[cut:])
    o, lse = A.merge_state_pair(va, la, vb, lb)
    o_ref, lse_ref = _state(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)
    # the merge does not care which state comes first
    o2, lse2 = A.merge_state_pair(vb, lb, va, la)
    np.testing.assert_allclose(o2, o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)


def test_row_major_states_over_a_scattered_key_split():
    """S = 6 states per (row, head) in the [R, S, H, D] layout, each over a
    scattered subset of the keys, one of them empty with NaN in its v."""
    rng = np.random.default_rng(47)
    R, H, L, S = 5, 3, 301, 6
    q, k, v = _qkv(rng, R, H, L)
    owner = rng.integers(0, S - 1, L)  # state S-1 owns no key
    vs = np.empty((R, S, H, D))
    ls = np.empty((R, S, H))
    for s in range(S):
        sel = np.flatnonzero(owner == s)
        if sel.size == 0:
            vs[:, s] = np.nan
            ls[:, s] = -np.inf
        else:
            vs[:, s], ls[:, s] = _state(q, k[sel], v[sel])
    o, lse = A.merge_state_rows(vs, ls)
    assert o.shape == (R, H, D) and lse.shape == (R, H)
    o_ref, lse_ref = _state(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(48)
    va = rng.standard_normal((4, 2, D))
    vb = rng.standard_normal((4, 2, D))
    la = rng.standard_normal((4, 2)) * 3
    # equal lse: the mean, and lse + ln 2
    o, lse = A.merge_state_pair(va, la, vb, la)
    np.testing.assert_allclose(o, (va + vb) / 2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, la + math.log(2.0), rtol=1e-15)
    # an empty partner drops out even when its v is NaN
    nan = np.full_like(vb, np.nan)
    empty = np.full_like(la, -np.inf)
    o, lse = A.merge_state_pair(va, la, nan, empty)
    assert np.array_equal(o, va) and np.array_equal(lse, la)
    o, lse = A.merge_state_pair(nan, empty, va, la)
    assert np.array_equal(o, va) and np.array_equal(lse, la)
    # all empty: zero output, -inf lse
    o, lse = A.merge_state_pair(nan, empty, nan, empty)
    assert not o.any() and np.isneginf(lse).all()
    # one state: unchanged
    o, lse = A.merge_state_rows(va[:, None], la[:, None])
    assert np.array_equal(o, va) and np.array_equal(lse, la)
    # weights: a state 20 nats above the other dominates by e^20
    o, lse = A.merge_state_pair(va, la + 20.0, vb, la)
    w = 1.0 / (1.0 + math.exp(-20.0))
    np.testing.assert_allclose(o, w * va + (1 - w) * vb, rtol=1e-13, atol=1e-15)
