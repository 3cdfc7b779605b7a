"""Helpers for the GPU parity tests: device copies and the acceptance checks."""
import sys

import numpy as np
import torch

from oracle import bf16

# BF16 attention outputs vs the float64 oracle: max |err| <= 2e-2 and
# ||err||_2 / ||ref||_2 <= 5e-3 (the acceptance bounds stated for this path).
MAX_ABS = 2e-2
REL_L2 = 5e-3


def note(msg):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a):
    """numpy uint16 (bf16 bits) / int32 / float32 -> contiguous CUDA tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def host(t):
    return t.cpu().numpy()


def assert_attention_close(got_bits, ref_f64, what=""):
    got = bf16.to_f64(got_bits)
    assert got.shape == ref_f64.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - ref_f64
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref_f64), 1e-30))
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=2e-4, err_msg=what)
