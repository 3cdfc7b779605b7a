"""Guard bytes around everything the entry points write.

Each output, status array, workspace and (for the appends) KV pool lives in
the middle of a larger buffer whose first and last 4 KiB hold a canary
pattern.  After each call the canaries must be intact, so no kernel writes
before or past the regions the C ABI describes; the outputs are also checked
against the oracle so the call did its work.  Decode runs in both modes at
P = 1 and P > 1, ragged and paged prefill with and without the key split,
both appends, both merges and both standalone RoPE forms.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import rope as R
from tests.gpu_helpers import assert_attention_close, dev, host, host_bits, note
from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


class Guarded:
    """A tensor of `shape`/`dtype` with canary bytes on both sides."""

    def __init__(self, shape, dtype, init=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = n
        self.buf = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(init)

    def intact(self):
        return bool((self.buf[:GUARD] == CANARY).all().item() and
                    (self.buf[GUARD + self.nbytes:] == CANARY).all().item())


def guarded_like(host_array):
    t = dev(host_array)
    return Guarded(tuple(t.shape), t.dtype, t)


def check_guards(**named):
    torch.cuda.synchronize()
    bad = [k for k, g in named.items() if g is not None and not g.intact()]
    assert not bad, f"canary bytes overwritten around: {bad}"


@pytest.mark.parametrize("mode", ["direct", "balanced"])
@pytest.mark.parametrize("P", [1, 3])
def test_decode_writes_inside_its_regions(mode, P):
    lens = [1, 17, 300, 2000, 999, 64]
    case = W.decode_case(901 + P, batch=len(lens), num_qo_heads=32, num_kv_heads=8,
                         seq_lens=lens, num_partitions=P, poison=True)
    ensure_built()
    kv = case.kv
    B, hq, _ = case.q.shape
    o = Guarded((B, hq, 128), torch.int16)
    lse = Guarded((B, hq), torch.float32)
    st = Guarded((B,), torch.int32)
    nb = (oxa.oxa_paged_decode_balanced_workspace_bytes(B, hq, P) if mode == "balanced"
          else oxa.oxa_paged_decode_workspace_bytes(B, hq, P))
    ws = Guarded((nb,), torch.uint8) if nb else None
    note(f"guards: decode {mode} P={P}")
    rc = oxa.oxa_paged_decode(dev(case.q), dev(kv.k_pool), dev(kv.v_pool), dev(kv.page_indptr),
                              dev(kv.page_indices), dev(kv.seq_lens), o.t,
                              max_seq_len=case.max_seq_len, sm_scale=case.sm_scale,
                              layout=kv.layout, num_kv_heads=kv.num_kv_heads, num_partitions=P,
                              workspace=None if ws is None else ws.t.view(torch.float32),
                              lse=lse.t, status=st.t)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    check_guards(o=o, lse=lse, status=st, workspace=ws)
    assert (host(st.t) == 0).all()
    o_ref, _ = A.paged_decode(case.q, kv.k_pool, kv.v_pool, kv.layout, kv.page_indptr,
                              kv.page_indices, kv.seq_lens, case.sm_scale)
    assert_attention_close(host_bits(o.t), o_ref, f"decode {mode} P={P}")


@pytest.mark.parametrize("split", [False, True])
def test_ragged_prefill_writes_inside_its_regions(split):
    qo = [1, 33, 64, 130, 257]
    case = W.ragged_case(911, qo_lens=qo, kv_lens=[5, 40, 64, 700, 300], num_qo_heads=8,
                         num_kv_heads=2)
    ensure_built()
    n, hq = case.q.shape[0], case.q.shape[1]
    o = Guarded((n, hq, 128), torch.int16)
    lse = Guarded((n, hq), torch.float32)
    st = Guarded((len(qo),), torch.int32)
    ws = None
    if split:
        nb = oxa.oxa_ragged_prefill_workspace_bytes(len(qo), n, hq)
        assert nb > 0
        ws = Guarded((nb,), torch.uint8)
    note(f"guards: ragged prefill split={split}")
    rc = oxa.oxa_ragged_prefill(dev(case.q), dev(case.k), dev(case.v), dev(case.qo_indptr),
                                dev(case.kv_indptr), o.t, max_qo_len=max(qo), max_kv_len=700,
                                sm_scale=case.sm_scale, causal=True, lse=lse.t, status=st.t,
                                workspace=None if ws is None else ws.t)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    check_guards(o=o, lse=lse, status=st, workspace=ws)
    assert (host(st.t) == 0).all()
    o_ref, _ = A.ragged_prefill(case.q, case.k, case.v, case.qo_indptr, case.kv_indptr,
                                case.sm_scale, True)
    assert_attention_close(host_bits(o.t), o_ref, f"ragged split={split}")


@pytest.mark.parametrize("split", [False, True])
def test_paged_prefill_writes_inside_its_regions(split):
    case = W.pages_paged_gqa4(poison=True)
    kv = case.kv
    ensure_built()
    n, hq = case.q.shape[0], case.q.shape[1]
    o = Guarded((n, hq, 128), torch.int16)
    lse = Guarded((n, hq), torch.float32)
    st = Guarded((2,), torch.int32)
    ws = None
    if split:
        nb = oxa.oxa_paged_prefill_workspace_bytes(2, n, hq)
        assert nb > 0
        ws = Guarded((nb,), torch.uint8)
    note(f"guards: paged prefill split={split}")
    rc = oxa.oxa_paged_prefill(dev(case.q), dev(case.qo_indptr), dev(kv.k_pool), dev(kv.v_pool),
                               dev(kv.page_indptr), dev(kv.page_indices), dev(kv.seq_lens), o.t,
                               max_qo_len=64, max_seq_len=1024, sm_scale=case.sm_scale,
                               layout=kv.layout, num_kv_heads=kv.num_kv_heads, causal=True,
                               lse=lse.t, status=st.t, workspace=None if ws is None else ws.t)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    check_guards(o=o, lse=lse, status=st, workspace=ws)
    assert host(st.t).tolist() == [0, 0]
    o_ref, _ = A.paged_prefill(case.q, case.qo_indptr, kv.k_pool, kv.v_pool, kv.layout,
                               kv.page_indptr, kv.page_indices, kv.seq_lens, case.sm_scale, True)
    assert_attention_close(host_bits(o.t), o_ref, f"paged split={split}")


@pytest.mark.parametrize("fused", [True, False])
def test_appends_write_inside_their_regions(fused):
    case = W.append_case(921, seq_lens=[5, 40, 130], num_qo_heads=8, num_kv_heads=2,
                         spare_pages=3)
    kv = case.kv
    ensure_built()
    nnz = case.k.shape[0]
    kp, vp = guarded_like(kv.k_pool), guarded_like(kv.v_pool)
    st = Guarded((2,), torch.int32)
    nb = (oxa.oxa_paged_append_rope_workspace_bytes(nnz) if fused
          else oxa.oxa_paged_append_workspace_bytes(nnz))
    ws = Guarded((nb,), torch.uint8)
    q_out = Guarded(case.q.shape, torch.int16) if fused else None
    note(f"guards: append fused={fused}")
    args = (dev(case.k), dev(case.v), dev(case.batch_indices), dev(case.positions), kp.t, vp.t,
            dev(kv.page_indptr), dev(kv.page_indices), dev(case.page_refcounts), st.t)
    if fused:
        rc = oxa.oxa_paged_append_rope(dev(case.q), q_out.t, *args, layout=kv.layout,
                                       rope_theta=case.rope_theta, workspace=ws.t)
    else:
        rc = oxa.oxa_paged_append(*args, layout=kv.layout, workspace=ws.t)
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    check_guards(k_pages=kp, v_pages=vp, status=st, workspace=ws, q_out=q_out)
    assert host(st.t).tolist() == [0, -1]
    if fused:
        reason, q_ref, k_ref, v_ref = R.paged_append_rope(
            case.q, case.k, case.v, case.batch_indices, case.positions, kv.k_pool, kv.v_pool,
            kv.layout, kv.page_indptr, kv.page_indices, case.page_refcounts, case.rope_theta)
        assert reason is None
        assert np.array_equal(host_bits(q_out.t), q_ref)
        assert np.array_equal(host_bits(kp.t), k_ref) and np.array_equal(host_bits(vp.t), v_ref)


@pytest.mark.parametrize("dout", [torch.int16, torch.float32])
def test_merges_write_inside_their_regions(dout):
    Rr, S, H = 37, 5, 6
    case = W.merge_case(931, Rr, S, H, dtype="f32")
    ensure_built()
    v, lse = dev(case.v), dev(case.lse)
    o = Guarded((Rr, H, 128), dout)
    lo = Guarded((Rr, H), torch.float32)
    note("guards: merge_states")
    assert oxa.oxa_merge_states(v, lse, o.t, lo.t) == oxa.OXA_OK
    check_guards(v_out=o, lse_out=lo)
    o_ref, _ = A.merge_state_rows(np.asarray(case.v, np.float64), case.lse)
    got = host_bits(o.t) if dout == torch.int16 else host(o.t)
    if dout == torch.int16:
        assert_attention_close(got, o_ref, "merge_states")
    else:
        np.testing.assert_allclose(got, o_ref, rtol=1e-5, atol=1e-5)
    # the pair merge, out of place
    a, b = v[:, 0].contiguous(), v[:, 1].contiguous()
    la, lb = lse[:, 0].contiguous(), lse[:, 1].contiguous()
    o2 = Guarded((Rr, H, 128), dout)
    lo2 = Guarded((Rr, H), torch.float32)
    note("guards: merge_state_pair")
    assert oxa.oxa_merge_state_pair(a, la, b, lb, o2.t, lo2.t) == oxa.OXA_OK
    check_guards(v_out=o2, lse_out=lo2)


@pytest.mark.parametrize("form", ["neox", "llama31"])
def test_rope_writes_inside_its_regions(form):
    rng = np.random.default_rng(941)
    nnz, hq, hkv = 77, 8, 2
    q = W.bf16_normal(rng, (nnz, hq, 128))
    k = W.bf16_normal(rng, (nnz, hkv, 128))
    pos = rng.integers(0, 100000, size=nnz).astype(np.int32)
    ensure_built()
    qo = Guarded(q.shape, torch.int16)
    ko = Guarded(k.shape, torch.int16)
    note(f"guards: rope {form}")
    if form == "neox":
        rc = oxa.oxa_rope_neox(dev(q), qo.t, dev(k), ko.t, dev(pos), rope_theta=10000.0)
        want_q = R.rope_neox_bf16(q, pos, 10000.0)
    else:
        rc = oxa.oxa_rope_llama31(dev(q), qo.t, dev(k), ko.t, dev(pos), rope_theta=500000.0)
        want_q = None
    assert rc == oxa.OXA_OK, oxa.status_string(rc)
    check_guards(q_out=qo, k_out=ko)
    if want_q is not None:
        assert np.array_equal(host_bits(qo.t), want_q)
