"""bf16 <-> float64 conversions for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits and 7
stored fraction bits (8 significant bits for normal numbers).  Storage in this
package is ``uint16`` bit patterns.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly (via the binary32 they extend)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def from_f64(x) -> np.ndarray:
    """Round float64 values to bf16, nearest with ties to even, in one step.

    The quantum of a finite value is 2**(e-8) where x = m * 2**e with
    0.5 <= |m| < 1 (eight significant bits), floored at 2**-133, the bf16
    subnormal spacing.  ``np.rint`` rounds half to even.  Values whose rounded
    magnitude exceeds the largest finite bf16 become infinities; NaN maps to a
    quiet NaN.  Rounding straight from float64 avoids the double rounding of a
    float64 -> float32 -> bf16 chain.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum_exp = np.maximum(e.astype(np.int64) - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -quantum_exp)), quantum_exp)
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isinf(x), x, r)
        f32 = r.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)
