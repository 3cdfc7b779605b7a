"""NeoX rotary embedding and the fused RoPE + paged KV append (test infrastructure only).

Pages cited: "Oxide Infer" README, section "Operator surface" (Position: BF16
NeoX RoPE with explicit positions; KV cache: RoPE plus paged append), and
"FlashInfer parity matrix", section "Admitted attention matrix" (Standard RoPE:
D128 NeoX split-half with explicit I32 positions, recorded through position
32,767; Fused RoPE plus paged append: explicit tokens with per-page reference
counts) and section "Paged KV ownership difference" (append writes only to pages
whose reference count is one; the pager makes targets private beforehand).

Readings of points the pages leave open:

* Frequencies: inv_freq_i = theta ** (-2 i / D), i = 0 .. D/2 - 1, theta given
  by the caller (10000 in the benchmark workload); all D dims rotate.
* Split-half pairing: dims (i, i + D/2) form the pair; with angle a = pos *
  inv_freq_i the rotated pair is (x_i cos a - x_{i+D/2} sin a,
  x_{i+D/2} cos a + x_i sin a).
* One int32 position per token serves both as the RoPE position and as the
  token's logical KV slot within its sequence.
* The fused op also rotates Q when a Q tensor is given (rotated Q is what the
  following prefill reads); V is stored unrotated.
* Rotation happens in float64 from the bf16 inputs and is rounded to bf16 once.
* Standalone RoPE (the Standard RoPE row) rotates q and k of each token at its
  explicit position; any int32 position is allowed (a negative one rotates
  backwards).
* The Llama 3.1 variant ("Domain coverage", RoPE: standard, Llama 3.1 and
  fused variants; the pages name it and give no formula) is taken as the
  published Llama 3.1 frequency rule: with the standard table f_i and
  wavelength w_i = 2 pi / f_i, frequencies whose wavelength is shorter than
  original_max_position / high_freq_factor stay, those longer than
  original_max_position / low_freq_factor are divided by factor, and those in
  between blend the two linearly in original_max_position / w_i.
* A call whose tokens break any rule writes nothing (all or nothing) and
  reports the first failing token's reason, checking per token in this order:
  "batch_index" (0 <= b < batch), "capacity" (0 <= pos < 16 * pages listed for
  b), "page_range" (target page id in [0, num_pages)), "not_exclusive" (target
  page's reference count is not exactly one).
"""
from __future__ import annotations

import numpy as np

from . import bf16

PAGE_SIZE = 16


def inv_freq(theta, head_dim):
    """theta ** (-2 i / D) for i = 0 .. D/2 - 1, float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * i / head_dim)


def inv_freq_llama31(theta, head_dim, factor, low_freq_factor, high_freq_factor,
                     original_max_position):
    """The Llama 3.1 rescaling of the standard frequency table, float64."""
    base = inv_freq(theta, head_dim)
    wavelen = 2.0 * np.pi / base
    low_freq_wavelen = original_max_position / low_freq_factor
    high_freq_wavelen = original_max_position / high_freq_factor
    smooth = (original_max_position / wavelen - low_freq_factor) / (
        high_freq_factor - low_freq_factor)
    blended = (1.0 - smooth) * base / factor + smooth * base
    out = np.where(wavelen > low_freq_wavelen, base / factor, blended)
    return np.where(wavelen < high_freq_wavelen, base, out)


def rope_neox(x, positions, theta, freqs=None):
    """Rotate float64 x [..., D] at integer positions [...] (NeoX split-half),
    with the standard table for theta or the given table ``freqs`` [D/2]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    table = inv_freq(theta, d) if freqs is None else np.asarray(freqs, np.float64)
    angle = np.asarray(positions, dtype=np.float64)[..., None] * table
    c, s = np.cos(angle), np.sin(angle)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_neox_bf16(x_bits, positions, theta, freqs=None):
    """bf16 in -> rotate in float64 -> bf16 out (one rounding)."""
    x = bf16.to_f64(x_bits)                               # [nnz, H, D]
    pos = np.asarray(positions)[:, None]                  # broadcast over heads
    return bf16.from_f64(rope_neox(x, pos, theta, freqs))


def append_status(batch_indices, positions, page_indptr, page_indices, page_refcounts,
                  num_pages, batch):
    """None if every token may be written, else (token, reason) of the first that may not."""
    for t in range(len(positions)):
        b = int(batch_indices[t])
        if b < 0 or b >= batch:
            return t, "batch_index"
        lo, hi = int(page_indptr[b]), int(page_indptr[b + 1])
        p = int(positions[t])
        if p < 0 or p >= (hi - lo) * PAGE_SIZE:
            return t, "capacity"
        page = int(page_indices[lo + p // PAGE_SIZE])
        if page < 0 or page >= num_pages:
            return t, "page_range"
        if int(page_refcounts[page]) != 1:
            return t, "not_exclusive"
    return None


def paged_append(k_bits, v_bits, batch_indices, positions, k_pool, v_pool, layout,
                 page_indptr, page_indices, page_refcounts):
    """Plain paged append ("Oxide Infer" README, "Operator surface": paged append
    beside RoPE plus paged append): (k, v) rows stored as they are, under the
    same all-or-nothing exclusive-page rules as the fused op.

    Returns (reason, k_pool_after, v_pool_after); on failure the pools come
    back unchanged.
    """
    batch = len(page_indptr) - 1
    bad = append_status(batch_indices, positions, page_indptr, page_indices,
                        page_refcounts, k_pool.shape[0], batch)
    if bad is not None:
        return bad[1], k_pool.copy(), v_pool.copy()
    k_after, v_after = _store(k_bits, v_bits, batch_indices, positions, k_pool, v_pool, layout,
                              page_indptr, page_indices)
    return None, k_after, v_after


def _store(k_rows, v_rows, batch_indices, positions, k_pool, v_pool, layout, page_indptr,
           page_indices):
    """Copies of the pools with token t's rows at (page, slot) of its position."""
    k_after, v_after = k_pool.copy(), v_pool.copy()
    for t in range(len(positions)):
        b, p = int(batch_indices[t]), int(positions[t])
        page = int(page_indices[int(page_indptr[b]) + p // PAGE_SIZE])
        slot = p % PAGE_SIZE
        if layout == "NHD":
            k_after[page, slot, :, :] = k_rows[t]
            v_after[page, slot, :, :] = v_rows[t]
        elif layout == "HND":
            k_after[page, :, slot, :] = k_rows[t]
            v_after[page, :, slot, :] = v_rows[t]
        else:
            raise ValueError(layout)
    return k_after, v_after


def paged_append_rope(q_bits, k_bits, v_bits, batch_indices, positions, k_pool, v_pool,
                      layout, page_indptr, page_indices, page_refcounts, theta):
    """Fused NeoX RoPE on q and k plus the append of (rotated k, v) into the pages.

    Returns (reason, q_out, k_pool_after, v_pool_after).  ``reason`` is None on
    success; otherwise the pools come back unchanged and q_out is None.
    """
    batch = len(page_indptr) - 1
    num_pages = k_pool.shape[0]
    bad = append_status(batch_indices, positions, page_indptr, page_indices,
                        page_refcounts, num_pages, batch)
    if bad is not None:
        return bad[1], None, k_pool.copy(), v_pool.copy()
    q_out = None if q_bits is None else rope_neox_bf16(q_bits, positions, theta)
    k_rot = rope_neox_bf16(k_bits, positions, theta)
    k_after, v_after = _store(k_rot, v_bits, batch_indices, positions, k_pool, v_pool, layout,
                              page_indptr, page_indices)
    return None, q_out, k_after, v_after
