"""Seeded synthetic inputs for paged BF16 attention.

This module only draws numbers and lays them out; it computes nothing that the
attention method computes.  The CPU oracle (``oracle/``) and the HIP library
(``paged_attention_02_amd``) both consume what it returns, and neither is
imported here.

Everything is numpy on the host:

* bf16 tensors are ``uint16`` bit patterns, drawn as float32 N(0, 1) and rounded
  to bf16 by torch's CPU cast (round-to-nearest-even);
* index tensors are ``int32``;
* a paged KV pool is one array per K and V.  Layout ``"NHD"`` is
  ``[num_pages, page_size, num_kv_heads, head_dim]`` and ``"HND"`` is
  ``[num_pages, num_kv_heads, page_size, head_dim]``.  Both hold the same
  values at the same (page, slot, head, dim) for a given seed.

The shapes follow the operator contracts of the "FlashInfer parity matrix"
page (section "Admitted attention matrix": BF16, head dim 128, page size 16,
NHD/HND paged rows) and the five benchmark workloads described there and on
the "Oxide Infer" README page (section "Performance snapshot").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

PAGE_SIZE = 16
HEAD_DIM = 128
NAN_BITS = np.uint16(0x7FC0)  # a quiet-NaN bf16 pattern used to poison unused slots


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) float32 samples rounded to bf16 (torch CPU cast, RNE); uint16 bits."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_layout(pool_nhd: np.ndarray, layout: str) -> np.ndarray:
    """Return a pool in the requested layout from its NHD form (a copy for HND)."""
    if layout == "NHD":
        return pool_nhd
    if layout == "HND":
        return np.ascontiguousarray(pool_nhd.transpose(0, 2, 1, 3))
    raise ValueError(layout)


def pages_for(lengths) -> np.ndarray:
    return np.array([(int(n) + PAGE_SIZE - 1) // PAGE_SIZE for n in lengths], dtype=np.int64)


def indptr_from_counts(counts) -> np.ndarray:
    out = np.zeros(len(counts) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(counts, dtype=np.int64))
    return out


@dataclasses.dataclass
class PagedKV:
    """A paged K/V pool plus the page table of one batch."""
    k_pool: np.ndarray          # uint16, layout-dependent 4-D shape
    v_pool: np.ndarray
    layout: str
    page_indptr: np.ndarray     # int32 [B + 1]
    page_indices: np.ndarray    # int32 [page_indptr[-1]]
    seq_lens: np.ndarray        # int32 [B]
    num_kv_heads: int

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])


def make_paged_kv(rng, seq_lens, num_kv_heads, *, num_pages=None, layout="NHD",
                  shuffle=True, poison=False, extra_pages=0) -> PagedKV:
    """Draw a pool and give each sequence ceil(len/16) distinct physical pages.

    ``shuffle`` draws the physical page ids as a random permutation of the pool
    (pages in arbitrary physical order); otherwise sequences take consecutive
    ids.  ``extra_pages`` appends that many additional pages to every sequence's
    list (capacity for appends) beyond what its length needs.  ``poison``
    overwrites every slot no sequence can see (unreferenced pages and the tail
    of each partial last page) with NaN bits.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = pages_for(seq_lens) + int(extra_pages)
    total = int(need.sum())
    if num_pages is None:
        num_pages = total
    assert num_pages >= total
    shape = (num_pages, PAGE_SIZE, num_kv_heads, HEAD_DIM)
    k = bf16_normal(rng, shape)
    v = bf16_normal(rng, shape)
    ids = rng.permutation(num_pages)[:total] if shuffle else np.arange(total)
    page_indices = ids.astype(np.int32)
    page_indptr = indptr_from_counts(need)
    if poison:
        visible = np.zeros((num_pages, PAGE_SIZE), dtype=bool)
        for b, n in enumerate(seq_lens):
            lo = int(page_indptr[b])
            for j in range(0, int(n), PAGE_SIZE):
                p = int(page_indices[lo + j // PAGE_SIZE])
                visible[p, : min(PAGE_SIZE, int(n) - j)] = True
        k[~visible] = NAN_BITS
        v[~visible] = NAN_BITS
    return PagedKV(to_layout(k, layout), to_layout(v, layout), layout,
                   page_indptr, page_indices, seq_lens, num_kv_heads)


# --------------------------------------------------------------------------
# The five benchmark workloads (scaled-down variants for parity use the same
# recipe with smaller sizes).  Seeds are 1000 + workload number.
# --------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeCase:
    q: np.ndarray               # uint16 [B, Hq, 128]
    kv: PagedKV
    num_qo_heads: int
    sm_scale: float
    num_partitions: int
    max_seq_len: int


def decode_case(seed, *, batch, num_qo_heads, num_kv_heads, seq_lens=None,
                seq_len_range=None, num_pages=None, layout="NHD", num_partitions=1,
                poison=False, shuffle=True) -> DecodeCase:
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        lo, hi = seq_len_range
        seq_lens = rng.integers(lo, hi, size=batch, endpoint=True)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    kv = make_paged_kv(rng, seq_lens, num_kv_heads, num_pages=num_pages, layout=layout,
                       poison=poison, shuffle=shuffle)
    q = bf16_normal(rng, (batch, num_qo_heads, HEAD_DIM))
    return DecodeCase(q, kv, num_qo_heads, 1.0 / math.sqrt(HEAD_DIM), num_partitions,
                      int(seq_lens.max()))


def decode_mha_small(poison=False, layout="NHD") -> DecodeCase:
    """Single-sequence MHA decode: 4 heads, kv_len 256, 16 pages permuted in a 64-page pool."""
    return decode_case(1001, batch=1, num_qo_heads=4, num_kv_heads=4, seq_lens=[256],
                       num_pages=64, layout=layout, poison=poison)


def decode_gqa4_batch(poison=False, layout="NHD", num_partitions=1, batch=32,
                      seq_len_range=(512, 4096)) -> DecodeCase:
    """Batch-32 GQA4 decode, 32 q / 8 kv heads, seq_lens uniform in [512, 4096]."""
    return decode_case(1002, batch=batch, num_qo_heads=32, num_kv_heads=8,
                       seq_len_range=seq_len_range, layout=layout, poison=poison,
                       num_partitions=num_partitions)


def decode_skewed(poison=False, layout="NHD") -> DecodeCase:
    """Skewed batch-32 GQA4 decode: one 32768-token sequence and 31 of 1024
    (32 q / 8 kv heads), the case load balancing is for."""
    return decode_case(1010, batch=32, num_qo_heads=32, num_kv_heads=8,
                       seq_lens=[32768] + [1024] * 31, layout=layout, poison=poison)


def decode_mqa_long(poison=False, layout="NHD", seq_len=32768, batch=8,
                    num_partitions=16) -> DecodeCase:
    """Long MQA decode: batch 8, 32 q heads / 1 kv head, seq_len 32768, 16 KV partitions."""
    return decode_case(1003, batch=batch, num_qo_heads=32, num_kv_heads=1,
                       seq_lens=[seq_len] * batch, layout=layout, poison=poison,
                       num_partitions=num_partitions)


@dataclasses.dataclass
class RaggedCase:
    q: np.ndarray               # uint16 [nnz_qo, Hq, 128]
    k: np.ndarray               # uint16 [nnz_kv, Hkv, 128]
    v: np.ndarray
    qo_indptr: np.ndarray       # int32 [B + 1]
    kv_indptr: np.ndarray       # int32 [B + 1]
    num_qo_heads: int
    num_kv_heads: int
    sm_scale: float
    causal: bool


def ragged_case(seed, *, qo_lens, kv_lens=None, num_qo_heads, num_kv_heads,
                causal=True) -> RaggedCase:
    rng = np.random.default_rng(seed)
    kv_lens = qo_lens if kv_lens is None else kv_lens
    qo_indptr = indptr_from_counts(qo_lens)
    kv_indptr = indptr_from_counts(kv_lens)
    q = bf16_normal(rng, (int(qo_indptr[-1]), num_qo_heads, HEAD_DIM))
    k = bf16_normal(rng, (int(kv_indptr[-1]), num_kv_heads, HEAD_DIM))
    v = bf16_normal(rng, (int(kv_indptr[-1]), num_kv_heads, HEAD_DIM))
    return RaggedCase(q, k, v, qo_indptr, kv_indptr, num_qo_heads, num_kv_heads,
                      1.0 / math.sqrt(HEAD_DIM), causal)


def ragged_gqa4_prefill(lengths=(512, 1024, 2048, 4096)) -> RaggedCase:
    """Ragged causal GQA4 prefill over sequences {512, 1024, 2048, 4096}, 32 q / 8 kv heads."""
    return ragged_case(1004, qo_lens=list(lengths), num_qo_heads=32, num_kv_heads=8)


@dataclasses.dataclass
class AppendCase:
    q: np.ndarray               # uint16 [nnz, Hq, 128]
    k: np.ndarray               # uint16 [nnz, Hkv, 128]
    v: np.ndarray
    batch_indices: np.ndarray   # int32 [nnz]
    positions: np.ndarray       # int32 [nnz]
    kv: PagedKV                 # pools to append into (contents are the "before" state)
    page_refcounts: np.ndarray  # int32 [num_pages]
    num_qo_heads: int
    rope_theta: float
    qo_indptr: np.ndarray       # int32 [B + 1]: tokens of sequence b in the nnz arrays
    sm_scale: float


def append_case(seed, *, seq_lens, num_qo_heads, num_kv_heads, layout="NHD",
                extra_pages=0, spare_pages=0, sentinel=True, rope_theta=10000.0) -> AppendCase:
    """Prefill-style append: every token 0..len-1 of each sequence, in order.

    The target pages are exclusive (refcount 1, each listed once), shuffled in
    a pool of ``sum(pages) + spare_pages`` pages.  With ``sentinel`` the pools
    start filled with a recognisable bit pattern so untouched slots can be
    checked bit for bit.
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = pages_for(seq_lens) + int(extra_pages)
    num_pages = int(need.sum()) + int(spare_pages)
    kv = make_paged_kv(rng, seq_lens, num_kv_heads, num_pages=num_pages, layout=layout,
                       extra_pages=extra_pages)
    if sentinel:
        kv.k_pool[...] = np.uint16(0x5A5A)
        kv.v_pool[...] = np.uint16(0xA5A5)
    nnz = int(seq_lens.sum())
    q = bf16_normal(rng, (nnz, num_qo_heads, HEAD_DIM))
    k = bf16_normal(rng, (nnz, num_kv_heads, HEAD_DIM))
    v = bf16_normal(rng, (nnz, num_kv_heads, HEAD_DIM))
    batch_indices = np.repeat(np.arange(len(seq_lens), dtype=np.int32), seq_lens)
    positions = np.concatenate([np.arange(n, dtype=np.int32) for n in seq_lens])
    refcounts = np.zeros(num_pages, dtype=np.int32)
    refcounts[kv.page_indices] = 1
    return AppendCase(q, k, v, batch_indices, positions, kv, refcounts, num_qo_heads,
                      float(rope_theta), indptr_from_counts(seq_lens), 1.0 / math.sqrt(HEAD_DIM))


def rope_append_prefill(seq_len=16384, batch=2) -> AppendCase:
    """Fused NeoX RoPE + exclusive paged append of 2 x 16384 tokens (32 q / 8 kv heads),
    whose pages and rotated q then feed a paged causal GQA4 prefill."""
    return append_case(1005, seq_lens=[seq_len] * batch, num_qo_heads=32, num_kv_heads=8,
                       sentinel=False)


# ----------------------------------------------------------------------------
# The attention shapes printed in the Oxide Infer README, Performance snapshot:
# paged decode B1 / KV1, ragged prefill MHA Q16 / KV16, ragged and paged
# prefill GQA4 with Q 32+64 over KV 256+1024; head dim 128, NHD, page size 16.
# The pages print no head counts; these cases take 32 q heads (32 kv heads for
# MHA, 8 for GQA4), as the other workloads do.

PAGES_HQ = 32


def pages_decode_b1_kv1(layout="NHD", poison=False) -> DecodeCase:
    """Paged decode, MHA, one sequence holding a single key."""
    return decode_case(1006, batch=1, num_qo_heads=PAGES_HQ, num_kv_heads=PAGES_HQ,
                       seq_lens=[1], num_pages=4, layout=layout, poison=poison)


def pages_ragged_mha_q16() -> RaggedCase:
    """Ragged causal prefill, MHA, one sequence of 16 queries over 16 keys."""
    return ragged_case(1007, qo_lens=[16], kv_lens=[16], num_qo_heads=PAGES_HQ,
                       num_kv_heads=PAGES_HQ)


def pages_ragged_gqa4() -> RaggedCase:
    """Ragged causal prefill, GQA4: queries 32 + 64 at the end of keys 256 + 1024
    (bottom-right causal alignment)."""
    return ragged_case(1008, qo_lens=[32, 64], kv_lens=[256, 1024], num_qo_heads=PAGES_HQ,
                       num_kv_heads=PAGES_HQ // 4)


@dataclasses.dataclass
class PagedPrefillCase:
    q: np.ndarray               # uint16 [nnz_qo, Hq, 128]
    qo_indptr: np.ndarray       # int32 [B + 1]
    kv: PagedKV
    num_qo_heads: int
    sm_scale: float


def pages_paged_gqa4(layout="NHD", poison=False) -> PagedPrefillCase:
    """Paged causal prefill, GQA4: queries 32 + 64 over paged keys 256 + 1024."""
    rng = np.random.default_rng(1009)
    kv = make_paged_kv(rng, np.array([256, 1024], np.int32), PAGES_HQ // 4, layout=layout,
                       poison=poison, extra_pages=0)
    qo_indptr = indptr_from_counts([32, 64])
    q = bf16_normal(rng, (int(qo_indptr[-1]), PAGES_HQ, HEAD_DIM))
    return PagedPrefillCase(q, qo_indptr, kv, PAGES_HQ, 1.0 / math.sqrt(HEAD_DIM))


# ----------------------------------------------------------------------------
# Attention states for the state merge: random outputs and log-sum-exps (not
# the states of any real attention; the merge is defined for any such input).

@dataclasses.dataclass
class MergeCase:
    v: np.ndarray        # [R, S, H, 128]: uint16 bf16 bits, or float32
    lse: np.ndarray      # float32 [R, S, H]; -inf marks an empty state
    dtype: str           # "bf16" or "f32"


def merge_case(seed, rows, states, heads, dtype="bf16", empty_frac=0.2, all_empty_units=1,
               lse_scale=4.0) -> MergeCase:
    """States v ~ N(0, 1) (bf16 or f32), lse ~ N(0, lse_scale^2); a fraction of
    the states are empty (lse = -inf, v NaN) and the first ``all_empty_units``
    (row, head) units have no live state at all."""
    rng = np.random.default_rng(seed)
    shape = (rows, states, heads, HEAD_DIM)
    if dtype == "bf16":
        v = bf16_normal(rng, shape)
    else:
        v = rng.standard_normal(size=shape, dtype=np.float32)
    lse = (rng.standard_normal(size=(rows, states, heads)) * lse_scale).astype(np.float32)
    empty = rng.random((rows, states, heads)) < empty_frac
    for u in range(min(all_empty_units, rows * heads)):
        empty[u // heads, :, u % heads] = True
    lse[empty] = -np.inf
    v[empty] = NAN_BITS if dtype == "bf16" else np.float32(np.nan)
    return MergeCase(v, lse, dtype)
