"""IEEE binary16 (fp16) rounding from float64, written from the format (oracle; test infrastructure only).

The FP8 linear layer's output dtype follows its input (page "transformers/integrations/deepgemm.py",
``deepgemm_fp8_fp4_linear``: bf16 or fp16 activations, ``torch.empty(..., dtype=input.dtype)``).
For fp16 the reading is the same as for bf16: round to nearest, ties to even, applied once to the
float64 value.

binary16: 1 sign bit, 5 exponent bits (bias 15), 10 stored mantissa bits, so 11 significant bits;
the largest finite value is 65504 and subnormals have spacing 2**-24.
"""

from __future__ import annotations

import numpy as np

F16_MAX = 65504.0


def round_to_f16(x) -> np.ndarray:
    """Round float64 values to the nearest fp16 value (ties to even); returns float64.

    Magnitudes that round beyond 65504 become +-inf; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e2 = np.frexp(mag)
    exp = np.maximum(e2.astype(np.int64) - 1, -14)  # leading-bit exponent, floored at the smallest normal
    quantum = np.ldexp(1.0, (exp - 10).astype(np.int32))  # 10 fraction bits below the leading bit
    with np.errstate(invalid="ignore", over="ignore"):
        rounded = np.rint(mag / quantum) * quantum
        rounded = np.where(np.isfinite(mag) & (rounded > F16_MAX), np.inf, rounded)
        rounded = np.where(np.isnan(x), np.nan, rounded)
    return np.copysign(rounded, x)


def to_bits(x) -> np.ndarray:
    """Round float64 values to fp16 and return the 16-bit patterns (uint16)."""
    return round_to_f16(x).astype(np.float16).view(np.uint16)  # the cast is exact on fp16 values


def from_bits(bits) -> np.ndarray:
    """fp16 bit patterns (uint16) -> float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp(x) -> np.ndarray:
    """Spacing of fp16 values at |x| (float64): 2**(floor(log2|x|) - 10), at least 2**-24."""
    mag = np.abs(np.asarray(x, dtype=np.float64))
    _, e2 = np.frexp(mag)
    # zero is subnormal: its spacing is 2**-24 (frexp gives 0 the exponent 0)
    exp = np.where(mag == 0.0, -14, np.maximum(e2.astype(np.int64) - 1, -14))
    return np.ldexp(1.0, (exp - 10).astype(np.int32))
