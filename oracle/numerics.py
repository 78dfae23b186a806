"""Number formats and the activation used between the two looped layers.
TEST INFRASTRUCTURE ONLY (see the package header).

The pages fix neither bf16 nor the activation; both readings are recorded in
the design notes:
  * bf16 is the upper half of an IEEE-754 binary32 word, rounded to nearest,
    ties to even (the definition of the format);
  * GELU is the exact form x * Phi(x), Phi the standard normal CDF.

Parity pins (tests/test_oracle_numerics.py): bf16 rounding against torch's CPU
float32->bfloat16 conversion on every class of input (ties, subnormals,
overflow to infinity, NaN), GELU against torch's exact-erf GELU in float64
and against closed-form values (GELU(0) = 0, GELU(x) - GELU(-x) = x).
"""

from __future__ import annotations

import numpy as np
from scipy.special import erf


def bf16_round(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return them
    as float32 values.  NaN stays NaN; overflow goes to +-inf."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = np.where(nan, np.uint64(0x7FC00000), r).astype(np.uint32)
    return r.view(np.float32).reshape(f.shape)


def bf16_bits(x) -> np.ndarray:
    """The 16-bit patterns of bf16_round(x)."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


def gelu(x) -> np.ndarray:
    """Exact GELU in float64: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))
