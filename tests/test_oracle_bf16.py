"""Pins of the oracle's bf16 conversions against torch's casts and hand-derived cases."""
import numpy as np
import pytest
import torch

from oracle import bf16


def torch_f32_to_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_widening_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16.to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_rounding_matches_torch_on_binary32_inputs():
    # Every value here is a binary32, so torch's single RNE step is the reference.
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e38).astype(np.float32),    # near overflow
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    assert np.array_equal(bf16.from_f64(x.astype(np.float64)), torch_f32_to_bf16_bits(x))


def test_ties_go_to_even_and_no_double_rounding():
    one = 1.0
    ulp = 2.0 ** -7
    # exact halfway points: 1 + ulp/2 -> 1 (even); 1 + 3ulp/2 -> 1 + 2ulp (even)
    assert bf16.to_f64(bf16.from_f64(one + ulp / 2)) == one
    assert bf16.to_f64(bf16.from_f64(one + 1.5 * ulp)) == one + 2 * ulp
    # a float64 just above the tie rounds up, though its binary32 rounding is the tie
    x = one + ulp / 2 + 2.0 ** -40
    assert np.float32(x) == np.float32(one + ulp / 2)
    assert bf16.to_f64(bf16.from_f64(x)) == one + ulp
    # sign symmetry, zero, infinities, NaN
    assert bf16.from_f64(-0.0) == 0x8000 and bf16.from_f64(0.0) == 0
    assert bf16.from_f64(np.inf) == 0x7F80 and bf16.from_f64(-np.inf) == 0xFF80
    assert bf16.from_f64(3.5e38) == 0x7F80          # beyond the largest finite bf16
    assert np.isnan(bf16.to_f64(bf16.from_f64(np.nan)))
    assert bf16.from_f64(-(one + 1.5 * ulp)) == (bf16.from_f64(one + 1.5 * ulp) | 0x8000)


@pytest.mark.parametrize("bits", [0x3F80, 0x0001, 0x007F, 0x0080, 0x7F7F, 0xC2F7])
def test_round_trip_is_exact(bits):
    assert bf16.from_f64(bf16.to_f64(np.uint16(bits))) == bits
