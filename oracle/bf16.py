"""bf16 rounding from float64, written from the format's definition (oracle; test infrastructure only).

The output dtype is bf16 (page "prhub.com.cn ... vllm/pull/49932", section
"关键源码片段": ``out_dtype = torch.bfloat16``; page
"vllm-project/vllm/pull/19085": ``gemm_fp8_fp8_bf16_nt``). The pages do not
state the rounding; the reading taken is round to nearest, ties to even,
applied once to the float64 value (no intermediate float32 rounding, which
could round twice).

bf16: 1 sign bit, 8 exponent bits (bias 127, as float32), 7 stored mantissa
bits, so 8 significant bits; subnormals have spacing 2**-133.
"""

from __future__ import annotations

import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even); returns float64.

    Magnitudes that round beyond the largest finite bf16 become +-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e2 = np.frexp(mag)
    exp = np.maximum(e2.astype(np.int64) - 1, -126)  # leading-bit exponent, floored at the smallest normal
    quantum = np.ldexp(1.0, (exp - 7).astype(np.int32))  # 7 fraction bits below the leading bit
    with np.errstate(invalid="ignore", over="ignore"):
        rounded = np.rint(mag / quantum) * quantum
        rounded = np.where(np.isfinite(mag) & (rounded > _BF16_MAX), np.inf, rounded)
        rounded = np.where(np.isnan(x), np.nan, rounded)
    return np.copysign(rounded, x)


def to_bits(x) -> np.ndarray:
    """Round float64 values to bf16 and return the 16-bit patterns (uint16)."""
    r = round_to_bf16(x).astype(np.float32)  # exact: every bf16 value is a float32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def from_bits(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        return b.view(np.float32).astype(np.float64)


def ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (float64): 2**(floor(log2|x|) - 7), at least 2**-133."""
    mag = np.abs(np.asarray(x, dtype=np.float64))
    _, e2 = np.frexp(mag)
    # zero lies in the subnormal range, whose spacing is the smallest normal binade's (frexp
    # gives 0 the exponent 0, which would make its spacing 2**-8)
    exp = np.where(mag == 0.0, -126, np.maximum(e2.astype(np.int64) - 1, -126))
    return np.ldexp(1.0, (exp - 7).astype(np.int32))
