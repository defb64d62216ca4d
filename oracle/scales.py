"""Coarser scales expanded to the block grids (oracle; test infrastructure only).

Page "vllm/pull/19085" (the review thread on per-tensor FP8 models): a model quantized with one
scale per tensor can run on the block kernel once its scales are expanded to the block shape.
A per-tensor or per-token (one per row of A) scale is constant over every 1x128 activation group
and every 128x128 weight block it covers, so the expansion is exact: the block GEMM with the
expanded grids computes the per-tensor / per-token product

    C[m, n] = bf16( s_a[m] * s_b * sum_k dec(A[m, k]) * dec(B[n, k]) ).

A per-output-channel weight scale (one per row of B) varies inside a 128-row weight block and
has no block form; it is not expanded.
"""

from __future__ import annotations

import numpy as np

from . import bf16, e4m3

BLOCK = 128


def expand_act_scales_ref(s, m: int, k: int) -> np.ndarray:
    """[M, ceil(K/128)] block scales from one scale (shape ()) or one per row (shape [M])."""
    s = np.asarray(s, dtype=np.float32)
    col = np.broadcast_to(s.reshape(-1) if s.ndim else s, (m,))
    return np.repeat(col[:, None], -(-k // BLOCK), axis=1).astype(np.float32)


def expand_weight_scale_ref(s, n: int, k: int) -> np.ndarray:
    """[ceil(N/128), ceil(K/128)] block scales from one per-tensor scale."""
    return np.full((-(-n // BLOCK), -(-k // BLOCK)), np.float32(s), dtype=np.float32)


def gemm_per_token_ref(a_q, s_a, b_q, s_b) -> np.ndarray:
    """bf16 bits of C = s_a[m] * s_b * sum_k dec(A) dec(B): the plain FP8 product with a
    per-token (or, with a scalar s_a, per-tensor) activation scale and a per-tensor weight
    scale. Every product of two e4m3 values is a multiple of 2^-18 below 2^36 such units, so
    the dot products are exact in float64 for K <= 2^17; the scale product then rounds once."""
    a = e4m3.decode(np.asarray(a_q))
    b = e4m3.decode(np.asarray(b_q))
    dots = a @ b.T
    sa = np.broadcast_to(np.asarray(s_a, dtype=np.float64).reshape(-1), (a.shape[0],))
    return bf16.to_bits(dots * (sa[:, None] * np.float64(np.float32(s_b))))
