"""Blockwise-scaled FP8 GEMM, dense and M-grouped contiguous (oracle; test infrastructure only).

Definition (the ``native_w8a8_block_matmul`` reference of the vLLM test on page
"prhub.com.cn ... vllm/pull/49932", section "关键源码片段", with the block
contract of its "实现拆解" item 2: activation groups 1x128, weight blocks 128x128):

    C[m, n] = sum_kb  P_kb[m, n] * As[m, kb] * Bs[n // 128, kb]
    P_kb[m, n] = sum_{k in block kb} dec(A_q[m, k]) * dec(B_q[n, k])

A_q[M, K] and B_q[N, K] are e4m3fn codes, both K-contiguous ("NT": the test
calls ``_scaled_mm(A, B.t(), ...)``); As is float32 [M, ceil(K/128)] and Bs is
float32 [ceil(N/128), ceil(K/128)]. The result is rounded once to bf16.

Exactness: every e4m3 value is an integer multiple of 2**-9 whose integer is
below 2**18 in magnitude, so each product is a multiple of 2**-18 below 2**36
units of 2**-18, and any sum of at most 128 of them stays below 2**43 units:
float64 (53 bits) holds every partial sum of a block exactly, whatever the
order. So P_kb computed with a float64 matrix product is exact. The scale
product As*Bs of two float32 values is exact in float64; only the final sum
over blocks (at most a few hundred terms) rounds, at 2**-53 relative, far
below the bf16 output rounding.

1x64 / 128x64 layout (``k_block=64``): the vLLM torch-backend page ("实现拆解" lists the
1x128 / 128x128 contract; "风险与影响" names 1x64 activation groups and 128x64 weight blocks as
the next layouts). Read plainly, the same sum over K blocks of 64: As is [M, ceil(K/64)], Bs is
[ceil(N/128), ceil(K/64)] (weight blocks stay 128 rows tall), and P_kb sums 64 products, which
the exactness argument above covers a fortiori.

Grouped contiguous (page "transformers/integrations/deepgemm.py",
``_build_deepgemm_contiguous_layout`` and ``deepgemm_fp8_fp4_experts_forward``):
each row r carries a group id g = layout[r]; rows with g >= 0 are the dense
product with B[g], Bs[g]; rows with g == -1 are padding and have no defined
output.
"""

from __future__ import annotations

import numpy as np

from . import bf16, e4m3

BLOCK = 128


def _check_shapes(a_q, a_s, b_q, b_s, k_block=BLOCK):
    m, k = a_q.shape
    n, k2 = b_q.shape
    if k != k2:
        raise ValueError("A and B disagree on K")
    if k_block not in (64, 128):
        raise ValueError("k_block must be 128 or 64")
    kb = -(-k // k_block)
    if a_s.shape != (m, kb):
        raise ValueError(f"As must be [{m}, {kb}], got {a_s.shape}")
    if b_s.shape != (-(-n // BLOCK), kb):
        raise ValueError(f"Bs must be [{-(-n // BLOCK)}, {kb}], got {b_s.shape}")
    return m, n, k, kb


def gemm_acc_ref(a_q, a_s, b_q, b_s, rows=None, cols=None, k_block=BLOCK) -> tuple[np.ndarray, np.ndarray]:
    """Unrounded float64 result and the matching sum of absolute block terms.

    Returns (acc, absum), each [len(rows), len(cols)]:
      acc   = sum_kb P_kb * As * Bs
      absum = sum_kb |P_kb * As * Bs|   (size of the terms, for error bounds)
    ``rows``/``cols`` select a subset of output rows/columns (default: all); rows
    are independent of each other, so a subset is the same definition. ``k_block``
    is the K width of a scale block: 128, or 64 for the 1x64 / 128x64 layout.
    """
    a_q = np.asarray(a_q)
    b_q = np.asarray(b_q)
    a_s = np.asarray(a_s, dtype=np.float32)
    b_s = np.asarray(b_s, dtype=np.float32)
    m, n, k, n_kb = _check_shapes(a_q, a_s, b_q, b_s, k_block)
    rows = np.arange(m) if rows is None else np.asarray(rows)
    cols = np.arange(n) if cols is None else np.asarray(cols)
    a_val = e4m3.decode(a_q[rows])  # float64
    b_val = e4m3.decode(b_q[cols])
    a_sc = a_s[rows].astype(np.float64)  # [r, kb]
    b_sc = b_s[cols // BLOCK].astype(np.float64)  # [c, kb]: weight block row of each column
    acc = np.zeros((rows.size, cols.size), dtype=np.float64)
    absum = np.zeros_like(acc)
    for kb in range(n_kb):
        ks = slice(kb * k_block, min((kb + 1) * k_block, k))
        p = a_val[:, ks] @ b_val[:, ks].T  # exact (see module docstring)
        term = p * (a_sc[:, kb][:, None] * b_sc[:, kb][None, :])
        acc += term
        absum += np.abs(term)
    return acc, absum


def gemm_ref(a_q, a_s, b_q, b_s, rows=None, cols=None, k_block=BLOCK) -> np.ndarray:
    """bf16 bit patterns (uint16) of C = bf16(sum_kb P_kb * As * Bs)."""
    acc, _ = gemm_acc_ref(a_q, a_s, b_q, b_s, rows, cols, k_block)
    return bf16.to_bits(acc)


def grouped_gemm_contiguous_acc_ref(a_q, a_s, b_q, b_s, layout, rows=None, cols=None):
    """M-grouped contiguous product: float64 acc and absum for rows with layout >= 0.

    a_q [M, K], a_s [M, ceil(K/128)], b_q [G, N, K], b_s [G, ceil(N/128), ceil(K/128)],
    layout int32 [M] (group id per row, -1 = padding). Returns (rows, acc, absum)
    where ``rows`` lists the non-padding rows considered (in increasing order).
    """
    layout = np.asarray(layout)
    b_q = np.asarray(b_q)
    b_s = np.asarray(b_s)
    g_count = b_q.shape[0]
    all_rows = np.arange(layout.shape[0]) if rows is None else np.asarray(rows)
    valid = all_rows[layout[all_rows] >= 0]
    if (layout[valid] >= g_count).any():
        raise ValueError("layout holds a group id >= G")
    n = b_q.shape[1]
    n_cols = n if cols is None else len(cols)
    acc = np.zeros((valid.size, n_cols), dtype=np.float64)
    absum = np.zeros_like(acc)
    for g in np.unique(layout[valid]):
        sel = np.nonzero(layout[valid] == g)[0]
        r = valid[sel]
        acc_g, abs_g = gemm_acc_ref(a_q, a_s, b_q[g], b_s[g], rows=r, cols=cols)
        acc[sel] = acc_g
        absum[sel] = abs_g
    return valid, acc, absum


def grouped_gemm_contiguous_ref(a_q, a_s, b_q, b_s, layout, rows=None, cols=None):
    """(rows, bf16 bits) of the grouped product for the non-padding rows."""
    valid, acc, _ = grouped_gemm_contiguous_acc_ref(a_q, a_s, b_q, b_s, layout, rows, cols)
    return valid, bf16.to_bits(acc)


def grouped_gemm_contiguous_nn_acc_ref(a_q, a_s, b_nn, bs_nn, layout, rows=None, cols=None):
    """The grouped product with NN expert weights (page "transformers/integrations/deepgemm.py",
    ``grouped_fp8_fp4_matmul_nn`` for ``is_transposed`` experts): b_nn [G, K, N] (N contiguous) and
    its scales bs_nn [G, ceil(K/128), ceil(N/128)]; C[m, n] = sum_kb sum_{k in kb} a[m, k] b_nn[g][k, n]
    * As[m, kb] * Bs_nn[g][kb, n // 128]. Returns (rows, acc) for the non-padding rows.

    Written on the NN operands directly: per expert, per K block, decoded codes multiplied with
    the K-major weight block as it is stored."""
    layout = np.asarray(layout)
    b_nn = np.asarray(b_nn)
    bs_nn = np.asarray(bs_nn, dtype=np.float32)
    a_q = np.asarray(a_q)
    a_s = np.asarray(a_s, dtype=np.float32)
    k = a_q.shape[1]
    n = b_nn.shape[2]
    all_rows = np.arange(layout.shape[0]) if rows is None else np.asarray(rows)
    valid = all_rows[layout[all_rows] >= 0]
    cols = np.arange(n) if cols is None else np.asarray(cols)
    acc = np.zeros((valid.size, cols.size), dtype=np.float64)
    for g in np.unique(layout[valid]):
        sel = np.nonzero(layout[valid] == g)[0]
        r = valid[sel]
        a_val = e4m3.decode(a_q[r])
        b_val = e4m3.decode(b_nn[g][:, cols])  # [K, cols]
        for kb in range(-(-k // BLOCK)):
            ks = slice(kb * BLOCK, min((kb + 1) * BLOCK, k))
            p = a_val[:, ks] @ b_val[ks, :]
            acc[sel] += p * (a_s[r, kb].astype(np.float64)[:, None] * bs_nn[g, kb, cols // BLOCK].astype(np.float64)[None, :])
    return valid, acc
