"""UE8M0 (power-of-two) scale factors (oracle; test infrastructure only).

Defined on page "transformers/integrations/deepgemm.py":
  * ``_ceil_to_ue8m0``: a float32 scale factor is rounded *up* to a power of two by
    adding 2**23 - 1 to its bit pattern and clearing the 23 mantissa bits (a value whose
    mantissa is already zero is unchanged);
  * ``_select_fp8_cast_kwargs``: FP8 weights with UE8M0 scale factors quantize their
    activations with ``use_ue8m0`` at gran_k = 128, i.e. the per-token-group float32
    scale of the ``quant`` module, rounded up to a power of two the same way;
  * ``_coerce_sf_for_kernel``: a ``float8_e8m0fnu`` scale is the biased exponent byte of
    a power-of-two float32, so byte e stands for 2**(e - 127) (byte 255 is NaN).

The quantizer of this module therefore takes the steps of ``quant.quant_act_ref`` with
one more: s = ceil_to_ue8m0(fl32(max(amax, 1e-10) / 448)), q = e4m3_RNE(clamp(fl32(x / s),
+-448)). Dividing by a power of two is exact, so the only rounding of the code is e4m3's.
The GEMM of UE8M0 operands is the blockwise GEMM of ``gemm`` with the decoded scales.
"""

from __future__ import annotations

import numpy as np

from . import e4m3, gemm
from .quant import AMAX_FLOOR, FP8_MAX, GROUP

MANTISSA_MASK = np.uint32((1 << 23) - 1)


def ceil_to_ue8m0(sf) -> np.ndarray:
    """float32 scale factors rounded up to powers of two through their bit patterns."""
    bits = np.asarray(sf, dtype=np.float32).view(np.uint32)
    with np.errstate(over="ignore"):
        up = (bits + MANTISSA_MASK) & ~MANTISSA_MASK
    return up.astype(np.uint32).view(np.float32)


def encode(pow2) -> np.ndarray:
    """UE8M0 code of power-of-two float32 values 2**-127 .. 2**127 (the biased exponent)."""
    bits = np.asarray(pow2, dtype=np.float32).view(np.uint32)
    smallest = bits == np.uint32(1 << 22)  # 2**-127, a float32 subnormal: code 0
    not_pow2 = ((bits & MANTISSA_MASK) != 0) & ~smallest
    if np.any(not_pow2) or np.any(bits >> 31) or np.any(bits == 0):
        raise ValueError("UE8M0 encodes positive powers of two 2**-127 .. 2**127 only")
    return np.where(smallest, 0, bits >> 23).astype(np.uint8)


def decode(codes) -> np.ndarray:
    """UE8M0 bytes -> float64 values 2**(e - 127); byte 255 is NaN."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("UE8M0 codes must be uint8")
    out = np.ldexp(1.0, codes.astype(np.int64) - 127)
    return np.where(codes == 255, np.nan, out)


def quant_act_ue8m0_ref(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize x[M, K] per 1x128 group with power-of-two scales.

    Returns (q, e): q uint8 e4m3fn codes [M, K]; e uint8 UE8M0 scale codes
    [M, ceil(K/128)] in row-major (m, group) order (the kernel ABI stores them group-major).
    """
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    x32 = x.astype(np.float32)  # bf16/fp16 -> fp32 is exact
    m, k = x32.shape
    n_groups = -(-k // GROUP)
    q = np.empty((m, k), dtype=np.uint8)
    e = np.empty((m, n_groups), dtype=np.uint8)
    with np.errstate(divide="raise", invalid="raise", over="raise", under="ignore"):
        for g in range(n_groups):
            cols = slice(g * GROUP, min((g + 1) * GROUP, k))
            xg = x32[:, cols]
            amax = np.abs(xg).max(axis=1) if m else np.zeros(0, np.float32)
            s32 = np.maximum(amax, AMAX_FLOOR) / FP8_MAX  # IEEE float32 division
            sg = ceil_to_ue8m0(s32)
            y = xg / sg[:, None]  # exact: sg is a power of two
            y = np.minimum(np.maximum(y, -FP8_MAX), FP8_MAX)
            q[:, cols] = e4m3.encode(y)
            e[:, g] = encode(sg)
    return q, e


def gemm_acc_ue8m0_ref(a_q, a_e, b_q, b_e, rows=None, cols=None):
    """(acc, absum) of the blockwise GEMM with UE8M0 scale codes a_e [M, KB], b_e [NB, KB]."""
    return gemm.gemm_acc_ref(a_q, decode(a_e).astype(np.float32), b_q, decode(b_e).astype(np.float32), rows, cols)
