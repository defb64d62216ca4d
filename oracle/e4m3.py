"""OCP float8 e4m3fn codec, written from the format's definition (oracle; test infrastructure only).

Page "prhub.com.cn ... vllm/pull/49932", section "关键源码片段": operands are
``torch.float8_e4m3fn`` with ``finfo`` max 448 and min -448, and the weights are
clamped to that range before the cast.

Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
  exponent field 0      -> subnormal, value = mantissa * 2**-9
  exponent field 1..15  -> normal,    value = (1 + mantissa/8) * 2**(exp - 7)
  0x7F and 0xFF         -> NaN (the "fn" variant has no infinities)
Largest finite magnitude: 0x7E = 1.75 * 2**8 = 448.

Encoding rounds to nearest with ties to even, keeps the sign of zero, and is
only defined here for |y| <= 448 (callers clamp first, as the page's recipe
does); a larger finite input raises.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6  # smallest normal exponent (field 1)


def _build_decode_table() -> np.ndarray:
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if (code & 0x7F) == 0x7F:
            table[code] = np.nan
        elif exp_field == 0:
            table[code] = sign * mant * 2.0**-9
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


DECODE_TABLE = _build_decode_table()
DECODE_TABLE.setflags(write=False)


def decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn byte codes (uint8, any shape) -> float64 values."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3 codes must be uint8")
    return DECODE_TABLE[codes]


def encode(y) -> np.ndarray:
    """Round values with |y| <= 448 to the nearest e4m3fn code (ties to even).

    ``y`` may be float32 or float64; each value is rounded once, exactly, from
    the value it holds. Returns uint8 codes of the same shape.
    """
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError("e4m3 encode: NaN input")
    mag = np.abs(y)
    if (mag > E4M3_MAX).any():
        raise ValueError("e4m3 encode: |y| > 448; clamp before encoding")
    # exponent of the leading bit: mag = f * 2**e2 with f in [0.5, 1) -> floor(log2 mag) = e2 - 1
    _, e2 = np.frexp(mag)
    exp = np.maximum(e2.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    exp = np.where(mag == 0.0, _MIN_NORMAL_EXP, exp)
    # spacing of representable values near mag: 3 mantissa bits below the leading bit;
    # the subnormal range shares the spacing of the smallest binade (2**-9)
    quantum = np.ldexp(1.0, (exp - 3).astype(np.int32))
    units = np.rint(mag / quantum)  # exact scaling by a power of two, then round half to even
    value = units * quantum  # the rounded magnitude (exactly representable in e4m3)
    # code of the rounded magnitude
    code = np.empty(mag.shape, dtype=np.int64)
    sub = value < 2.0**_MIN_NORMAL_EXP
    # subnormal (and zero): code = value / 2**-9  (0..7); value 2**-6 falls in the normal branch
    code[sub] = np.rint(value[sub] / 2.0**-9).astype(np.int64)
    nv = value[~sub]
    _, ve = np.frexp(nv)
    vexp = ve.astype(np.int64) - 1
    mant = np.rint(nv / np.ldexp(1.0, (vexp - 3).astype(np.int32))).astype(np.int64) - 8
    code[~sub] = ((vexp + 7) << 3) | mant
    sign = np.signbit(y).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def ulp(codes: np.ndarray) -> np.ndarray:
    """Spacing of e4m3 values at the magnitude of each (finite) code, in float64.

    2**(floor(log2|q|) - 3) for |q| >= 2**-6, else 2**-9 (the subnormal spacing).
    """
    v = np.abs(decode(codes))
    _, e2 = np.frexp(v)
    # zero is subnormal: its spacing is 2**-9 (frexp gives 0 the exponent 0)
    exp = np.where(v == 0.0, _MIN_NORMAL_EXP, np.maximum(e2.astype(np.int64) - 1, _MIN_NORMAL_EXP))
    return np.ldexp(1.0, (exp - 3).astype(np.int32))
