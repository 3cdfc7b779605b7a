"""Softmax attention over a paged KV cache, in float64 (test infrastructure only).

Pages cited: "FlashInfer parity matrix", section "Admitted attention matrix"
(rows Single decode split-K, Paged batch decode, Ragged causal prefill, Paged
causal prefill, and the note under the table: BF16, NHD layout, head dim 128,
page size 16, F32 softmax state, causal only where the row says so) and section
"Domain coverage" (NHD and HND paged layouts).  The method computes exactly
(up to rounding order) softmax attention, so this module is that definition
written out: scores, a maximum-shifted exponential, its sum, the weighted sum
of V and the log of the normaliser.  Nothing is blocked, fused or reordered.

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):

* A query head h reads KV head h // (Hq / Hkv) (contiguous head groups).
* Layouts: NHD pool = [page, slot, kv_head, dim]; HND pool = [page, kv_head,
  slot, dim]; K and V live in two separate pools.
* Logical token j of sequence b lives in physical page
  ``page_indices[page_indptr[b] + j // 16]`` at slot ``j % 16``; a sequence
  may list more pages than its length needs (capacity for appends); only the
  first ceil(len / 16) are read.
* Causal masking is aligned bottom-right: query row i of a sequence with
  qo_len query rows and kv_len keys sees keys j <= i + (kv_len - qo_len).
* The log-sum-exp is natural-log: lse = m + ln(sum_j exp(s_j - m)).
* Split-K ("explicit partitions"): partition p of a sequence covers the
  logical pages [p*C, (p+1)*C) with C = ceil(ceil(max_seq_len / 16) / P);
  an empty partition has state (O = 0, lse = -inf) and drops out of the merge.
"""
from __future__ import annotations

import numpy as np

from . import bf16

PAGE_SIZE = 16
HEAD_DIM = 128


# ---------------------------------------------------------------------------
# Page-table resolution
# ---------------------------------------------------------------------------

def gather(pool_bits, layout, page_indptr, page_indices, b, length) -> np.ndarray:
    """Rows 0..length-1 of sequence b from a paged pool, as float64 [length, Hkv, D].

    Logical row j -> page ``page_indices[page_indptr[b] + j // 16]``, slot
    ``j % 16`` ("FlashInfer parity matrix", Admitted attention matrix: paged
    rows with page size 16; Domain coverage: NHD/HND paged decode).
    """
    j = np.arange(int(length))
    page = np.asarray(page_indices)[int(page_indptr[b]) + j // PAGE_SIZE]
    slot = j % PAGE_SIZE
    pool = np.asarray(pool_bits)
    if layout == "NHD":
        rows = pool[page, slot, :, :]
    elif layout == "HND":
        rows = pool[page, :, slot, :]
    else:
        raise ValueError(layout)
    return bf16.to_f64(rows)


# ---------------------------------------------------------------------------
# The definition
# ---------------------------------------------------------------------------

def attend(q, k, v, sm_scale, causal, q_rows=None, qo_len=None):
    """Softmax attention of float64 query rows over float64 keys/values.

    q: [n, Hq, D] query rows; k, v: [L, Hkv, D].  ``q_rows`` gives the index of
    each query row within its sequence's qo_len query rows (default 0..n-1,
    qo_len = n).  With ``causal`` query row i sees keys j <= i + (L - qo_len);
    otherwise every key.  Returns (o [n, Hq, D], lse [n, Hq]).

    Per query row and head:  s_j = sm_scale * <q, k_j>;  m = max_j s_j;
    w_j = exp(s_j - m);  l = sum_j w_j;  o = (sum_j w_j v_j) / l;
    lse = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    if q_rows is None:
        q_rows = np.arange(n)
        qo_len = n
    q_rows = np.asarray(q_rows)
    o = np.zeros((n, hq, d))
    lse = np.full((n, hq), -np.inf)
    if causal:
        visible = np.arange(L)[None, :] <= (q_rows[:, None] + (L - qo_len))
    else:
        visible = np.ones((n, L), dtype=bool)
    for h in range(hq):
        kh = h // g
        s = sm_scale * (q[:, h, :] @ k[:, kh, :].T)
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.where(visible, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
        l = w.sum(axis=1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            o[:, h, :] = (w @ v[:, kh, :]) / l
            lse[:, h] = (m + np.log(l))[:, 0]
    return o, lse


# ---------------------------------------------------------------------------
# Paged batch decode (+ split-K partials and their merge)
# ---------------------------------------------------------------------------

def decode_status(seq_lens, page_indptr, num_page_entries, page_indices, num_pages,
                  max_seq_len):
    """Per-sequence validity of decode metadata: None, or the first failing check.

    Checks in order: "seq_len" (1 <= len <= max_seq_len), "indptr"
    (0 <= indptr[b] <= indptr[b+1] <= number of page entries, and enough pages
    for the length), "page_range" (every page the length needs lies in
    [0, num_pages)).  A rejected call is a typed device-status failure in the
    pages' runtime model ("Oxide Infer" README, section "Providers": typed
    device-status failures; "FlashInfer parity matrix": invalid-page rejection
    in the Paged causal prefill Graph evidence).
    """
    out = []
    for b, n in enumerate(np.asarray(seq_lens)):
        n = int(n)
        lo, hi = int(page_indptr[b]), int(page_indptr[b + 1])
        if n < 1 or n > max_seq_len:
            out.append("seq_len")
        elif lo < 0 or hi < lo or hi > num_page_entries or (hi - lo) * PAGE_SIZE < n:
            out.append("indptr")
        else:
            need = (n + PAGE_SIZE - 1) // PAGE_SIZE
            ids = np.asarray(page_indices[lo:lo + need])
            out.append("page_range" if np.any((ids < 0) | (ids >= num_pages)) else None)
    return out


def paged_decode(q_bits, k_pool, v_pool, layout, page_indptr, page_indices, seq_lens,
                 sm_scale):
    """Paged batch decode: one query token per sequence over its whole paged KV.

    ("FlashInfer parity matrix", Admitted attention matrix, row Paged batch
    decode: MHA, MQA, GQA, mixed lengths, page order, read-only page reuse.)
    Returns float64 (o [B, Hq, D], lse [B, Hq]).
    """
    q = bf16.to_f64(q_bits)
    B, hq, d = q.shape
    o = np.zeros((B, hq, d))
    lse = np.zeros((B, hq))
    for b in range(B):
        L = int(seq_lens[b])
        k = gather(k_pool, layout, page_indptr, page_indices, b, L)
        v = gather(v_pool, layout, page_indptr, page_indices, b, L)
        ob, lb = attend(q[b:b + 1], k, v, sm_scale, causal=False)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def partition_pages(max_seq_len, num_partitions):
    """Pages per split-K partition: C = ceil(ceil(max_seq_len / 16) / P)."""
    pages = -(-int(max_seq_len) // PAGE_SIZE)
    return -(-pages // int(num_partitions))


def decode_partials(q_bits, k_pool, v_pool, layout, page_indptr, page_indices, seq_lens,
                    sm_scale, num_partitions, max_seq_len):
    """Split-K decode partial states per partition.

    ("FlashInfer parity matrix", Admitted attention matrix, row Single decode
    split-K: explicit partitions with an F32 partial workspace and a merge.)
    Partition p of sequence b attends over its tokens
    [p*C*16, min((p+1)*C*16, len)); its state is the normalised partial output
    o_p and lse_p; an empty partition is (0, -inf).
    Returns (o_part [B, Hq, P, D], lse_part [B, Hq, P]) in float64.
    """
    q = bf16.to_f64(q_bits)
    B, hq, d = q.shape
    P = int(num_partitions)
    C = partition_pages(max_seq_len, P)
    o_part = np.zeros((B, hq, P, d))
    lse_part = np.full((B, hq, P), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        k = gather(k_pool, layout, page_indptr, page_indices, b, L)
        v = gather(v_pool, layout, page_indptr, page_indices, b, L)
        for p in range(P):
            lo, hi = p * C * PAGE_SIZE, min((p + 1) * C * PAGE_SIZE, L)
            if lo >= hi:
                continue
            op, lp = attend(q[b:b + 1], k[lo:hi], v[lo:hi], sm_scale, causal=False)
            o_part[b, :, p, :] = op[0]
            lse_part[b, :, p] = lp[0]
    return o_part, lse_part


def merge_states(o_part, lse_part):
    """Combine partial attention states along the second-to-last axis of o_part.

    lse = ln sum_p exp(lse_p);  o = sum_p exp(lse_p - lse) * o_p.  A state with
    lse_p = -inf (an empty key set) contributes nothing, whatever its o_p holds;
    if every state is empty the result is (o = 0, lse = -inf).  (The merge of
    the Single decode split-K row; the "Attention state and cascade" domain's
    state merge.)
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    m = np.max(lse_part, axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_part - m_safe)
    total = np.sum(w, axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = (m_safe + np.log(total))[..., 0]
    live = ~np.isneginf(lse_part)
    frac = np.where(live, w / np.where(total > 0, total, 1.0), 0.0)
    o = np.sum(np.where(live[..., None], frac[..., None] * o_part, 0.0), axis=-2)
    return o, lse


def merge_state_rows(v, lse):
    """The state-merge operator over row-major states: v [R, S, H, D] and lse
    [R, S, H] (S states of each (row, head)) -> v [R, H, D], lse [R, H]."""
    v = np.asarray(v, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    return merge_states(np.transpose(v, (0, 2, 1, 3)), np.transpose(lse, (0, 2, 1)))


def merge_state_pair(v_a, lse_a, v_b, lse_b):
    """Two states of every (row, head): v [R, H, D], lse [R, H] each."""
    v = np.stack([np.asarray(v_a, np.float64), np.asarray(v_b, np.float64)], axis=-2)
    lse = np.stack([np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)], axis=-1)
    return merge_states(v, lse)


# ---------------------------------------------------------------------------
# Causal prefill, ragged and paged
# ---------------------------------------------------------------------------

def ragged_status(qo_indptr, kv_indptr, nnz_qo, nnz_kv, max_qo_len, max_kv_len, causal):
    """Per-sequence validity of ragged prefill metadata (None or first failing check).

    "indptr": both indptr arrays non-decreasing from >= 0 and within nnz;
    "seq_len": qo_len <= max_qo_len, kv_len <= max_kv_len, and kv_len >= 1 when
    qo_len >= 1; "causal": causal with qo_len > kv_len (no key visible to the
    first rows under bottom-right alignment).
    """
    out = []
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        if q0 < 0 or q1 < q0 or q1 > nnz_qo or k0 < 0 or k1 < k0 or k1 > nnz_kv:
            out.append("indptr")
            continue
        ql, kl = q1 - q0, k1 - k0
        if ql > max_qo_len or kl > max_kv_len or (ql > 0 and kl < 1):
            out.append("seq_len")
        elif causal and ql > kl:
            out.append("causal")
        else:
            out.append(None)
    return out


def ragged_prefill(q_bits, k_bits, v_bits, qo_indptr, kv_indptr, sm_scale, causal,
                   rows=None):
    """Ragged (packed) prefill: sequence b's queries q[qo_indptr[b]:qo_indptr[b+1]]
    attend to k/v[kv_indptr[b]:kv_indptr[b+1]].

    ("FlashInfer parity matrix", Admitted attention matrix, row Ragged causal
    prefill.)  ``rows`` optionally restricts the computation to those packed
    query rows (each row's result does not depend on the others).
    Returns (o [nnz_qo, Hq, D], lse [nnz_qo, Hq]); rows not computed are NaN.
    """
    nnz_qo, hq, d = q_bits.shape
    o = np.full((nnz_qo, hq, d), np.nan)
    lse = np.full((nnz_qo, hq), np.nan)
    want = np.ones(nnz_qo, dtype=bool) if rows is None else np.isin(np.arange(nnz_qo), rows)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        sel = np.nonzero(want[q0:q1])[0]
        if sel.size == 0:
            continue
        k = bf16.to_f64(k_bits[k0:k1])
        v = bf16.to_f64(v_bits[k0:k1])
        q = bf16.to_f64(q_bits[q0 + sel])
        ob, lb = attend(q, k, v, sm_scale, causal, q_rows=sel, qo_len=q1 - q0)
        o[q0 + sel], lse[q0 + sel] = ob, lb
    return o, lse


def paged_prefill_status(qo_indptr, nnz_qo, seq_lens, page_indptr, num_page_entries,
                         page_indices, num_pages, max_qo_len, max_seq_len, causal):
    """Per-sequence validity of paged prefill metadata (None or first failing check).

    Order: "indptr" (qo_indptr and page_indptr ranges), "seq_len"
    (qo_len <= max_qo_len, 0 <= kv_len <= max_seq_len, kv_len >= 1 when
    qo_len >= 1), "indptr" again if the sequence lists too few pages for kv_len,
    "causal" (qo_len > kv_len), "page_range" (a needed page id outside the pool).
    """
    out = []
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        p0, p1 = int(page_indptr[b]), int(page_indptr[b + 1])
        n = int(seq_lens[b])
        if q0 < 0 or q1 < q0 or q1 > nnz_qo or p0 < 0 or p1 < p0 or p1 > num_page_entries:
            out.append("indptr")
            continue
        ql = q1 - q0
        if ql > max_qo_len or n < 0 or n > max_seq_len or (ql > 0 and n < 1):
            out.append("seq_len")
        elif (p1 - p0) * PAGE_SIZE < n:
            out.append("indptr")
        elif causal and ql > n:
            out.append("causal")
        else:
            need = (n + PAGE_SIZE - 1) // PAGE_SIZE
            ids = np.asarray(page_indices[p0:p0 + need])
            out.append("page_range" if np.any((ids < 0) | (ids >= num_pages)) else None)
    return out


def paged_prefill(q_bits, qo_indptr, k_pool, v_pool, layout, page_indptr, page_indices,
                  seq_lens, sm_scale, causal, rows=None):
    """Paged prefill: sequence b's queries attend to its first seq_lens[b] paged
    tokens.  ("FlashInfer parity matrix", Admitted attention matrix, row Paged
    causal prefill.)  Same return convention as ``ragged_prefill``.
    """
    nnz_qo, hq, d = q_bits.shape
    o = np.full((nnz_qo, hq, d), np.nan)
    lse = np.full((nnz_qo, hq), np.nan)
    want = np.ones(nnz_qo, dtype=bool) if rows is None else np.isin(np.arange(nnz_qo), rows)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        sel = np.nonzero(want[q0:q1])[0]
        if sel.size == 0:
            continue
        L = int(seq_lens[b])
        k = gather(k_pool, layout, page_indptr, page_indices, b, L)
        v = gather(v_pool, layout, page_indptr, page_indices, b, L)
        q = bf16.to_f64(q_bits[q0 + sel])
        ob, lb = attend(q, k, v, sm_scale, causal, q_rows=sel, qo_len=q1 - q0)
        o[q0 + sel], lse[q0 + sel] = ob, lb
    return o, lse
