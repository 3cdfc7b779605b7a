"""Test-side constructions used to pin the oracle (never used by the HIP path)."""
import numpy as np
import torch
import torch.nn.functional as F

PAGE = 16


def sdpa(q, k, v, scale, causal):
    """torch's scaled_dot_product_attention in float64 on the CPU.

    q [n, Hq, D], k/v [L, Hkv, D] float64; KV heads are repeated to the query
    heads in contiguous groups.  torch's causal mask is aligned top-left, so it
    is only used here with n == L.
    """
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q)).permute(1, 0, 2)
    kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(g, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(g, dim=1).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


def torch_lse(q, k, scale):
    """torch.logsumexp over torch-computed logits, [n, Hq]."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q)).permute(1, 0, 2)
    kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(g, dim=1).permute(1, 0, 2)
    logits = scale * torch.matmul(qt, kt.transpose(1, 2))
    return torch.logsumexp(logits, dim=-1).permute(1, 0).numpy()


def scatter_pages(seqs, num_pages, layout, rng, extra_pages=0, fill=None):
    """Place logical per-sequence rows [L_b, H, D] (uint16) into a shuffled pool.

    Returns (pool, page_indptr, page_indices).  Unused slots hold ``fill`` bits
    (default: a NaN pattern).
    """
    h, d = seqs[0].shape[1], seqs[0].shape[2]
    counts = [-(-len(s) // PAGE) + extra_pages for s in seqs]
    assert sum(counts) <= num_pages
    ids = rng.permutation(num_pages)[: sum(counts)].astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pool = np.full((num_pages, PAGE, h, d), 0x7FC0 if fill is None else fill, dtype=np.uint16)
    for b, s in enumerate(seqs):
        for j in range(len(s)):
            pool[ids[indptr[b] + j // PAGE], j % PAGE] = s[j]
    if layout == "HND":
        pool = np.ascontiguousarray(pool.transpose(0, 2, 1, 3))
    return pool, indptr, ids
