"""Python binding of liboxa: BF16 attention over a paged KV cache on MI355X (gfx950).

The functions below carry the names of the C ABI declared in ``include/oxa.h``
and do argument marshalling only: they take torch tensors that live on the GPU
(bf16 tensors as ``torch.bfloat16`` or ``torch.int16``/``uint16`` views,
indices as ``torch.int32``), pass their device pointers and the current HIP
stream to the library and return its status code.  Every step of the
computation runs in the library's kernels; if the library cannot be loaded the
call raises.

Status codes: ``OXA_OK`` (0); host-detected errors ``OXA_ERR_*`` (returned at
once, nothing enqueued); device-detected ``OXA_DEV_*`` codes land in the
``status`` tensor after the stream completes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# the built library; OXA_LIBRARY names another build of it (a sanitized host layer, say)
LIB_PATH = os.environ.get("OXA_LIBRARY") or os.path.join(_HERE, "liboxa.so")

OXA_OK = 0
OXA_ERR_NULL = 1
OXA_ERR_UNSUPPORTED = 2
OXA_ERR_SHAPE = 3
OXA_ERR_ALIGN = 4
OXA_ERR_ALIAS = 5
OXA_ERR_WORKSPACE = 6
OXA_ERR_LAUNCH = 7
OXA_ERR_SCRATCH_LIMIT = 8
OXA_DECODE_SCRATCH_BYTES = 8 << 20
OXA_DEV_PAGE_RANGE = 16
OXA_DEV_INDPTR = 17
OXA_DEV_SEQ_LEN = 18
OXA_DEV_CAUSAL = 19
OXA_DEV_NOT_EXCLUSIVE = 20
OXA_DEV_CAPACITY = 21
OXA_DEV_BATCH_INDEX = 22

LAYOUTS = {"NHD": 0, "HND": 1}
OXA_DTYPE_BF16 = 0
OXA_DTYPE_F32 = 1
PAGE_SIZE = 16
HEAD_DIM = 128

# C signatures: (name, restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "oxa_abi_version": (_I, []),
    "oxa_status_string": (ctypes.c_char_p, [_I]),
    "oxa_paged_append_rope": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _P, _P, _I, _P, _P, _I, _I, _I,
                                   _P, _I, _P, _I, _P, _F, _P, _Z, _P]),
    "oxa_paged_append_rope_workspace_bytes": (_Z, [_I]),
    "oxa_paged_append": (_I, [_P, _P, _P, _I, _I, _P, _P, _I, _P, _P, _I, _I, _I, _P, _I, _P, _I,
                              _P, _P, _Z, _P]),
    "oxa_paged_append_workspace_bytes": (_Z, [_I]),
    "oxa_paged_decode": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _I, _P, _I, _F,
                              _I, _P, _Z, _P, _P, _P]),
    "oxa_paged_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "oxa_paged_decode_balanced_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "oxa_paged_decode_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _I, _P,
                                      _I, _F, _I, _P, _P, _P]),
    "oxa_ragged_prefill": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                _P, _Z, _P, _P, _P]),
    "oxa_ragged_prefill_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "oxa_paged_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                               _I, _I, _I, _F, _P, _Z, _P, _P, _P]),
    "oxa_paged_prefill_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "oxa_merge_states": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P]),
    "oxa_merge_state_pair": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P]),
    "oxa_rope_neox": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _P, _I, _F]),
    "oxa_rope_llama31": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _P, _I, _F, _F, _F, _F, _I]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded liboxa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"liboxa.so not found at {LIB_PATH}; build it with "
                "`python -m paged_attention_02_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(code: int) -> str:
    return lib().oxa_status_string(int(code)).decode()


class OxaError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"{status_string(code)} ({code})")
        self.code = code


def check(code: int) -> None:
    if code != OXA_OK:
        raise OxaError(code)


# ------------------------------------------------------------------ marshalling
#
# These run on every call, so they avoid per-call imports and Python-level
# stream objects: for a latency-bound launch the marshalling is a large part of
# the host time.

_torch = None
_BF16_DTYPES = ()


def _t():
    """torch, imported on first use (the module loads without it)."""
    global _torch, _BF16_DTYPES
    if _torch is None:
        import torch
        _torch = torch
        _BF16_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)
    return _torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, _t().Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _bf16(t, name):
    if t is not None:
        _t()
        if t.dtype not in _BF16_DTYPES:
            raise TypeError(f"{name} must be bf16 (or its 16-bit bit pattern)")
    return _ptr(t)


def _i32(t, name):
    if t is not None and t.dtype != _t().int32:
        raise TypeError(f"{name} must be int32")
    return _ptr(t)


def _f32(t, name):
    if t is not None and t.dtype != _t().float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t)


def _state_dtype(t, name) -> int:
    """oxa_dtype of an attention-state tensor: bf16 (or its bits) or float32."""
    torch = _t()
    if t.dtype in _BF16_DTYPES:
        return OXA_DTYPE_BF16
    if t.dtype == torch.float32:
        return OXA_DTYPE_F32
    raise TypeError(f"{name} must be bf16 or float32")


def _shape(t, shape, name):
    # torch.Size is a tuple: it compares with a tuple as it is
    if t is not None and t.shape != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _pools(k_pages, v_pages, lay, hkv=None):
    """Check a K/V pool pair: [pages, 16, Hkv, 128] (NHD) or [pages, Hkv, 16, 128]
    (HND), V shaped as K; returns Hkv."""
    if k_pages.dim() != 4:
        raise ValueError(f"k_pages must have 4 dimensions, got shape {tuple(k_pages.shape)}")
    heads = k_pages.shape[2] if lay == 0 else k_pages.shape[1]
    slots = k_pages.shape[1] if lay == 0 else k_pages.shape[2]
    if slots != PAGE_SIZE:
        raise ValueError(f"k_pages holds {slots} slots per page, expected {PAGE_SIZE}")
    if hkv is not None and heads != hkv:
        raise ValueError(f"k_pages holds {heads} kv heads, expected {hkv}")
    _shape(v_pages, k_pages.shape, "v_pages")
    return heads


def _no_alloc_under_capture(what):
    if _t().cuda.is_current_stream_capturing():
        raise RuntimeError(f"{what}: pass `workspace` when capturing a graph "
                           "(the binding would otherwise allocate one inside the capture)")


def _stream(stream) -> int:
    """The raw HIP stream: `stream`'s, else the current stream of the current
    device (read without building a torch Stream object, which costs more than
    a small kernel launch; the public call where that entry is missing)."""
    torch = _t()
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    dev = getattr(torch._C, "_cuda_getDevice", None)
    if raw is not None and dev is not None:
        return raw(dev())
    return torch.cuda.current_stream().cuda_stream


def _layout(layout) -> int:
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


# ------------------------------------------------------------------ entry points

def oxa_paged_append_rope_workspace_bytes(nnz) -> int:
    return int(lib().oxa_paged_append_rope_workspace_bytes(nnz))


def oxa_paged_append_rope(q_in, q_out, k_in, v_in, batch_indices, positions, k_pages, v_pages,
                          page_indptr, page_indices, page_refcounts, status, *, layout="NHD",
                          rope_theta=10000.0, workspace=None, stream=None) -> int:
    """Fused NeoX RoPE on q/k and append of (rotated k, v) into exclusive pages.

    q_in/q_out [nnz, Hq, 128] (both None to skip q), k_in/v_in [nnz, Hkv, 128],
    pools in ``layout``, status int32 [2] (code, first failing token).  Without
    a ``workspace`` tensor one of oxa_paged_append_rope_workspace_bytes(nnz)
    bytes is allocated on k_in's device.
    """
    lay = _layout(layout)
    nnz, hkv = k_in.shape[0], k_in.shape[1]
    num_pages = k_pages.shape[0]
    hq = q_in.shape[1] if q_in is not None else 0
    if q_in is not None:
        _shape(q_in, (nnz, hq, k_in.shape[2]), "q_in")
        _shape(q_out, q_in.shape, "q_out")
    elif q_out is not None:
        raise ValueError("q_out given without q_in")
    _shape(v_in, k_in.shape, "v_in")
    _shape(batch_indices, (nnz,), "batch_indices")
    _shape(positions, (nnz,), "positions")
    _pools(k_pages, v_pages, lay, hkv)
    _shape(page_refcounts, (num_pages,), "page_refcounts")
    _shape(status, (2,), "status")
    if workspace is None:
        import torch
        _no_alloc_under_capture("oxa_paged_append_rope")
        nbytes = oxa_paged_append_rope_workspace_bytes(k_in.shape[0])
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=k_in.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    return lib().oxa_paged_append_rope(
        _stream(stream), _bf16(q_in, "q_in"), _bf16(q_out, "q_out"), hq, _bf16(k_in, "k_in"),
        _bf16(v_in, "v_in"), hkv, k_in.shape[2], _i32(batch_indices, "batch_indices"),
        _i32(positions, "positions"), k_in.shape[0], _bf16(k_pages, "k_pages"),
        _bf16(v_pages, "v_pages"), num_pages, PAGE_SIZE, lay, _i32(page_indptr, "page_indptr"),
        page_indptr.shape[0] - 1, _i32(page_indices, "page_indices"), page_indices.shape[0],
        _i32(page_refcounts, "page_refcounts"), float(rope_theta), _ptr(workspace), ws_bytes,
        _i32(status, "status"))


def oxa_paged_append_workspace_bytes(nnz) -> int:
    return int(lib().oxa_paged_append_workspace_bytes(nnz))


def oxa_paged_append(k_in, v_in, batch_indices, positions, k_pages, v_pages, page_indptr,
                     page_indices, page_refcounts, status, *, layout="NHD", workspace=None,
                     stream=None) -> int:
    """Plain append of (k, v) rows into exclusive pages, no rotation; arguments
    as for oxa_paged_append_rope without q and rope_theta."""
    lay = _layout(layout)
    nnz = k_in.shape[0]
    _shape(v_in, k_in.shape, "v_in")
    _shape(batch_indices, (nnz,), "batch_indices")
    _shape(positions, (nnz,), "positions")
    _pools(k_pages, v_pages, lay, k_in.shape[1])
    _shape(page_refcounts, (k_pages.shape[0],), "page_refcounts")
    _shape(status, (2,), "status")
    if workspace is None:
        import torch
        _no_alloc_under_capture("oxa_paged_append")
        nbytes = oxa_paged_append_workspace_bytes(k_in.shape[0])
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=k_in.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    return lib().oxa_paged_append(
        _stream(stream), _bf16(k_in, "k_in"), _bf16(v_in, "v_in"), k_in.shape[1], k_in.shape[2],
        _i32(batch_indices, "batch_indices"), _i32(positions, "positions"), k_in.shape[0],
        _bf16(k_pages, "k_pages"), _bf16(v_pages, "v_pages"), k_pages.shape[0], PAGE_SIZE, lay,
        _i32(page_indptr, "page_indptr"), page_indptr.shape[0] - 1,
        _i32(page_indices, "page_indices"), page_indices.shape[0],
        _i32(page_refcounts, "page_refcounts"), _ptr(workspace), ws_bytes, _i32(status, "status"))


def oxa_paged_decode_workspace_bytes(batch, num_qo_heads, num_partitions, head_dim=HEAD_DIM) -> int:
    return int(lib().oxa_paged_decode_workspace_bytes(batch, num_qo_heads, head_dim,
                                                      num_partitions))


def oxa_paged_decode_balanced_workspace_bytes(batch, num_qo_heads, num_partitions,
                                              head_dim=HEAD_DIM) -> int:
    """Workspace bytes of the load-balanced decode mode (0 if the shape has none).

    Its merge counters must be zero before the first call with a workspace;
    every call leaves them zero (a zero-filled workspace can be reused)."""
    return int(lib().oxa_paged_decode_balanced_workspace_bytes(batch, num_qo_heads, head_dim,
                                                              num_partitions))


def oxa_paged_decode(q, k_pages, v_pages, page_indptr, page_indices, seq_lens, o, *,
                     max_seq_len, sm_scale, layout="NHD", num_kv_heads=None, num_partitions=1,
                     workspace=None, lse=None, status=None, stream=None) -> int:
    """Paged batch decode: q/o [B, Hq, 128]; lse [B, Hq] f32; status [B] int32."""
    lay = _layout(layout)
    num_kv_heads = _pools(k_pages, v_pages, lay, num_kv_heads)
    B, hq = q.shape[0], q.shape[1]
    _shape(o, q.shape, "o")
    _shape(lse, (B, hq), "lse")
    _shape(status, (B,), "status")
    _shape(seq_lens, (B,), "seq_lens")
    _shape(page_indptr, (B + 1,), "page_indptr")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return lib().oxa_paged_decode(
        _stream(stream), _bf16(q, "q"), q.shape[0], q.shape[1], num_kv_heads, q.shape[2],
        _bf16(k_pages, "k_pages"), _bf16(v_pages, "v_pages"), k_pages.shape[0], PAGE_SIZE, lay,
        _i32(page_indptr, "page_indptr"), _i32(page_indices, "page_indices"),
        page_indices.shape[0], _i32(seq_lens, "seq_lens"), int(max_seq_len), float(sm_scale),
        int(num_partitions), _ptr(workspace), ws_bytes, _bf16(o, "o"), _f32(lse, "lse"),
        _i32(status, "status"))


def oxa_paged_decode_noalloc(q, k_pages, v_pages, page_indptr, page_indices, seq_lens, o, *,
                             max_seq_len, sm_scale, layout="NHD", num_kv_heads=None,
                             num_partitions=1, lse=None, status=None, stream=None) -> int:
    """oxa_paged_decode without a workspace: the split-K partial states go to
    the library's static per-GPU scratch (OXA_DECODE_SCRATCH_BYTES), so the
    call allocates nothing; calls that overlap on one GPU race on it."""
    lay = _layout(layout)
    num_kv_heads = _pools(k_pages, v_pages, lay, num_kv_heads)
    B, hq = q.shape[0], q.shape[1]
    _shape(o, q.shape, "o")
    _shape(lse, (B, hq), "lse")
    _shape(status, (B,), "status")
    _shape(seq_lens, (B,), "seq_lens")
    _shape(page_indptr, (B + 1,), "page_indptr")
    return lib().oxa_paged_decode_noalloc(
        _stream(stream), _bf16(q, "q"), B, hq, num_kv_heads, q.shape[2],
        _bf16(k_pages, "k_pages"), _bf16(v_pages, "v_pages"), k_pages.shape[0], PAGE_SIZE, lay,
        _i32(page_indptr, "page_indptr"), _i32(page_indices, "page_indices"),
        page_indices.shape[0], _i32(seq_lens, "seq_lens"), int(max_seq_len), float(sm_scale),
        int(num_partitions), _bf16(o, "o"), _f32(lse, "lse"), _i32(status, "status"))


def oxa_ragged_prefill_workspace_bytes(batch, nnz_qo, num_qo_heads, head_dim=HEAD_DIM) -> int:
    return int(lib().oxa_ragged_prefill_workspace_bytes(batch, nnz_qo, num_qo_heads, head_dim))


def oxa_paged_prefill_workspace_bytes(batch, nnz_qo, num_qo_heads, head_dim=HEAD_DIM) -> int:
    return int(lib().oxa_paged_prefill_workspace_bytes(batch, nnz_qo, num_qo_heads, head_dim))


def _ws(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def oxa_ragged_prefill(q, k, v, qo_indptr, kv_indptr, o, *, max_qo_len, max_kv_len, sm_scale,
                       causal=True, lse=None, status=None, workspace=None, stream=None) -> int:
    """Ragged prefill: q/o [nnz_qo, Hq, 128]; k/v [nnz_kv, Hkv, 128].  With a
    ``workspace`` of oxa_ragged_prefill_workspace_bytes(...) bytes, small calls
    split their keys over more CUs."""
    B = qo_indptr.shape[0] - 1
    _shape(kv_indptr, qo_indptr.shape, "kv_indptr")
    _shape(v, k.shape, "v")
    _shape(o, q.shape, "o")
    _shape(lse, (q.shape[0], q.shape[1]), "lse")
    _shape(status, (B,), "status")
    return lib().oxa_ragged_prefill(
        _stream(stream), _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"),
        _i32(qo_indptr, "qo_indptr"), _i32(kv_indptr, "kv_indptr"), qo_indptr.shape[0] - 1,
        q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2], int(max_qo_len),
        int(max_kv_len), int(bool(causal)), float(sm_scale), _ptr(workspace), _ws(workspace),
        _bf16(o, "o"),
        _f32(lse, "lse"), _i32(status, "status"))


def oxa_paged_prefill(q, qo_indptr, k_pages, v_pages, page_indptr, page_indices, seq_lens, o, *,
                      max_qo_len, max_seq_len, sm_scale, layout="NHD", num_kv_heads=None,
                      causal=True, lse=None, status=None, workspace=None, stream=None) -> int:
    """Paged prefill: q/o [nnz_qo, Hq, 128] over the paged K/V of each sequence
    (``workspace`` as for oxa_ragged_prefill)."""
    lay = _layout(layout)
    num_kv_heads = _pools(k_pages, v_pages, lay, num_kv_heads)
    B = qo_indptr.shape[0] - 1
    _shape(page_indptr, (B + 1,), "page_indptr")
    _shape(seq_lens, (B,), "seq_lens")
    _shape(o, q.shape, "o")
    _shape(lse, (q.shape[0], q.shape[1]), "lse")
    _shape(status, (B,), "status")
    return lib().oxa_paged_prefill(
        _stream(stream), _bf16(q, "q"), _i32(qo_indptr, "qo_indptr"), _bf16(k_pages, "k_pages"),
        _bf16(v_pages, "v_pages"), k_pages.shape[0], PAGE_SIZE, lay,
        _i32(page_indptr, "page_indptr"), _i32(page_indices, "page_indices"),
        page_indices.shape[0], _i32(seq_lens, "seq_lens"), qo_indptr.shape[0] - 1, q.shape[0],
        q.shape[1], num_kv_heads, q.shape[2], int(max_qo_len), int(max_seq_len),
        int(bool(causal)), float(sm_scale), _ptr(workspace), _ws(workspace), _bf16(o, "o"),
        _f32(lse, "lse"),
        _i32(status, "status"))


def oxa_merge_states(v, lse, v_out, lse_out=None, *, stream=None) -> int:
    """Merge S attention states per (row, head): v [R, S, H, 128] (bf16 or f32),
    lse [R, S, H] f32 -> v_out [R, H, 128] (bf16 or f32), lse_out [R, H] f32."""
    R, S, H, D = v.shape
    _shape(lse, (R, S, H), "lse")
    _shape(v_out, (R, H, D), "v_out")
    _shape(lse_out, (R, H), "lse_out")
    return lib().oxa_merge_states(
        _stream(stream), _ptr(v), _f32(lse, "lse"), _state_dtype(v, "v"), R, S, H, D, _ptr(v_out),
        _state_dtype(v_out, "v_out"), _f32(lse_out, "lse_out"))


def oxa_merge_state_pair(v_a, lse_a, v_b, lse_b, v_out, lse_out=None, *, stream=None) -> int:
    """Merge two attention states per (row, head): v_a, v_b [R, H, 128] (same
    dtype), lse_a, lse_b [R, H] f32 -> v_out [R, H, 128], lse_out [R, H]; v_out
    may be v_a or v_b itself (and lse_out lse_a or lse_b) for an in-place merge."""
    R, H, D = v_a.shape
    if v_b.dtype != v_a.dtype:
        raise TypeError("v_a and v_b must have the same dtype")
    _shape(v_b, (R, H, D), "v_b")
    _shape(lse_a, (R, H), "lse_a")
    _shape(lse_b, (R, H), "lse_b")
    _shape(v_out, (R, H, D), "v_out")
    _shape(lse_out, (R, H), "lse_out")
    return lib().oxa_merge_state_pair(
        _stream(stream), _ptr(v_a), _f32(lse_a, "lse_a"), _ptr(v_b), _f32(lse_b, "lse_b"),
        _state_dtype(v_a, "v_a"), R, H, D, _ptr(v_out), _state_dtype(v_out, "v_out"),
        _f32(lse_out, "lse_out"))


def _rope_args(q_in, q_out, k_in, k_out, positions):
    ref = q_in if q_in is not None else k_in
    if ref is None:
        raise ValueError("pass q_in/q_out, k_in/k_out or both")
    nnz, _, d = ref.shape
    hq = q_in.shape[1] if q_in is not None else 0
    hkv = k_in.shape[1] if k_in is not None else 0
    if q_in is not None:
        _shape(q_out, q_in.shape, "q_out")
    if k_in is not None:
        _shape(k_in, (nnz, hkv, d), "k_in")
        _shape(k_out, k_in.shape, "k_out")
    _shape(positions, (nnz,), "positions")
    return [_bf16(q_in, "q_in"), _bf16(q_out, "q_out"), hq, _bf16(k_in, "k_in"),
            _bf16(k_out, "k_out"), hkv, d, _i32(positions, "positions"), nnz]


def oxa_rope_neox(q_in, q_out, k_in, k_out, positions, *, rope_theta=10000.0, stream=None) -> int:
    """NeoX RoPE of q [nnz, Hq, 128] and/or k [nnz, Hkv, 128] at positions [nnz]
    (int32); pass None for both tensors of a skipped side; outputs may be the
    inputs themselves."""
    return lib().oxa_rope_neox(_stream(stream), *_rope_args(q_in, q_out, k_in, k_out, positions),
                               float(rope_theta))


def oxa_rope_llama31(q_in, q_out, k_in, k_out, positions, *, rope_theta=500000.0, factor=8.0,
                     low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192,
                     stream=None) -> int:
    """As oxa_rope_neox with the Llama 3.1 frequency table."""
    return lib().oxa_rope_llama31(_stream(stream),
                                  *_rope_args(q_in, q_out, k_in, k_out, positions),
                                  float(rope_theta), float(factor), float(low_freq_factor),
                                  float(high_freq_factor), int(original_max_position))
