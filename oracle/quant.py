"""Per-token-group FP8 quantizer (oracle; test infrastructure only).

Defined by ``per_token_group_quant_fp8(x, 128)`` in the vLLM test on page
"prhub.com.cn ... vllm/pull/49932" (section "关键源码片段") and by
``per_token_cast_to_fp8`` with gran_k=128 and float32 scale factors on page
"transformers/integrations/deepgemm.py" (``_select_fp8_cast_kwargs``). Each row m
of x is cut into groups of 128 consecutive columns (the last group may be
shorter: the pages size the scale grid with ceil(K/128)); each group gets one
float32 scale.

The pages print no formula for the scale. Readings taken (each listed with its
justification in the design notes):
  * scale  s = fl32(max(amax, 1e-10) / 448), amax = max |x| over the group,
    448 = finfo(float8_e4m3fn).max; the 1e-10 floor keeps an all-zero group
    finite (it then quantizes to zeros);
  * code   q = e4m3_RNE(clamp(fl32(x / s), -448, 448)), with a correctly
    rounded float32 division (not a multiply by 1/s);
  * dequantized value x ~ q * s (s is the multiplier, like ``weight_scale_inv``).
The input is widened to float32 first (exact for bf16 and fp16 inputs).

Group width. The pages define 1x128 groups; the vLLM torch-backend page ("prhub.com.cn ...
vllm/pull/49932", section "风险与影响") names 1x64 activation groups (with 128x64 weight
blocks) as the next layouts to support. ``group=64`` is that layout, read plainly: the same
scale and code definition over groups of 64 consecutive columns (ceil(K/64) scales per row).
"""

from __future__ import annotations

import numpy as np

from . import e4m3

GROUP = 128
FP8_MAX = np.float32(448.0)
AMAX_FLOOR = np.float32(1e-10)


def quant_act_ref(x, group: int = GROUP) -> tuple[np.ndarray, np.ndarray]:
    """Quantize x[M, K] per 1 x ``group`` group (128, or 64 for the 1x64 layout).

    Returns (q, s): q uint8 e4m3fn codes [M, K]; s float32 scales [M, ceil(K/group)]
    in row-major (m, group) order. The kernel ABI stores the same values
    group-major; that is a layout choice, not a different result.
    """
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    if group not in (64, 128):
        raise ValueError("group must be 128 or 64")
    x32 = x.astype(np.float32)  # bf16/fp16 -> fp32 is exact
    m, k = x32.shape
    n_groups = -(-k // group)
    q = np.empty((m, k), dtype=np.uint8)
    s = np.empty((m, n_groups), dtype=np.float32)
    with np.errstate(divide="raise", invalid="raise", over="raise"):
        for g in range(n_groups):
            cols = slice(g * group, min((g + 1) * group, k))
            xg = x32[:, cols]
            amax = np.abs(xg).max(axis=1) if m else np.zeros(0, np.float32)
            sg = np.maximum(amax, AMAX_FLOOR) / FP8_MAX  # IEEE float32 division
            y = xg / sg[:, None]  # IEEE float32 division, one rounding
            y = np.minimum(np.maximum(y, -FP8_MAX), FP8_MAX)
            q[:, cols] = e4m3.encode(y)
            s[:, g] = sg
    return q, s


def dequant_ref(q, s, group: int = GROUP) -> np.ndarray:
    """q * s per group, in float64 (for round-trip checks)."""
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float64)
    k = q.shape[1]
    scale_full = np.repeat(s, group, axis=1)[:, :k]
    return e4m3.decode(q) * scale_full
