"""Mixture-of-experts chain around the M-grouped contiguous GEMM (oracle; test infrastructure only).

Defined on page "transformers/integrations/deepgemm.py":
  * ``_dispatch_routed_input`` / ``_build_deepgemm_contiguous_layout``: the S = T * top_k
    (token, expert) pairs are ordered by expert; expert e gets a block of rows that starts on
    a multiple of ``alignment`` (its count rounded up), blocks in expert order, pairs placed
    at ``arange + cumulative_padding[expert]``; the buffer has the upper bound
    S + min(S, E) * (alignment - 1) rows (no device-to-host sync); each row carries its
    expert id, -1 on padding; expert ids equal to E (expert-parallel sentinels) are counted
    by no expert and placed in no expert block;
  * ``deepgemm_fp8_fp4_experts_forward``: quantize the routed activations per 1x128 group,
    grouped GEMM with the up (gate+up) weights into bf16, the gate activation, quantize
    again, grouped GEMM with the down weights into bf16, then combine;
  * ``_combine_routed_output``: each pair's output row times its router weight cast to the
    output dtype (bf16), sentinel rows zeroed, back to token order, summed over the top_k
    pairs of each token.

Readings where the page is silent (listed in the design notes):
  * order of the pairs inside an expert block: stable, by pair index (the page's torch.sort
    leaves equal keys unordered; the result of the chain does not depend on it);
  * ids outside [0, E) are sentinels like E itself (counted by no expert, output zero);
  * the gate activation (``_apply_gate``, not printed): SwiGLU on the bf16 up-projection
    output, first half gate, second half up: h = bf16(bf16(silu(gate)) * up), silu(x) =
    x / (1 + exp(-x)) rounded once to bf16 from its exact value (evaluated in float64);
  * the top-k sum: float32, pairs added in order j = 0 .. top_k-1, rounded once to bf16.
"""

from __future__ import annotations

import numpy as np

from . import bf16, gemm, quant


def padded_rows(s: int, e: int, align: int) -> int:
    """The page's upper bound on the padded buffer: S + min(S, E) * (alignment - 1)."""
    return s + min(s, e) * (align - 1)


def layout_ref(expert_ids, num_experts: int, align: int):
    """(row_of_pair [S], pair_of_row [M_pad], layout [M_pad], expert_start [E+1]) as int arrays.

    row_of_pair[p] is pair p's row, -1 for a sentinel; layout[r] is row r's expert, -1 on
    padding; pair_of_row[r] is the pair in row r, -1 on padding."""
    ids = np.asarray(expert_ids).reshape(-1).astype(np.int64)
    s = ids.size
    valid = (ids >= 0) & (ids < num_experts)
    counts = np.bincount(ids[valid], minlength=num_experts)
    aligned = -(-counts // align) * align
    start = np.concatenate([[0], np.cumsum(aligned)])
    m_pad = padded_rows(s, num_experts, align)
    row_of_pair = np.full(s, -1, dtype=np.int64)
    seen = np.zeros(num_experts, dtype=np.int64)
    for p in range(s):  # pair-index order: stable inside each expert
        if valid[p]:
            e = ids[p]
            row_of_pair[p] = start[e] + seen[e]
            seen[e] += 1
    layout = np.full(m_pad, -1, dtype=np.int64)
    pair_of_row = np.full(m_pad, -1, dtype=np.int64)
    placed = row_of_pair >= 0
    layout[row_of_pair[placed]] = ids[placed]
    pair_of_row[row_of_pair[placed]] = np.nonzero(placed)[0]
    return row_of_pair, pair_of_row, layout, start


def silu_bf16_bits(gate_bits) -> np.ndarray:
    """bf16(silu(g)) from bf16 bits, silu evaluated in float64 and rounded once."""
    g = bf16.from_bits(np.asarray(gate_bits)).astype(np.float64)
    with np.errstate(over="ignore"):
        y = g / (1.0 + np.exp(-g))
    return bf16.to_bits(y)


def swiglu_ref(proj_bits) -> np.ndarray:
    """h = bf16(bf16(silu(gate)) * up) from the bf16 bits of [rows, 2I] (gate first, then up)."""
    proj_bits = np.asarray(proj_bits)
    i = proj_bits.shape[1] // 2
    s = bf16.from_bits(silu_bf16_bits(proj_bits[:, :i])).astype(np.float64)
    up = bf16.from_bits(proj_bits[:, i:]).astype(np.float64)
    return bf16.to_bits(s * up)  # the product of two bf16 values is exact in float64


def combine_ref(out_bits, row_of_pair, topk_weights, num_tokens: int, top_k: int) -> np.ndarray:
    """y [T, H] bf16 bits: per token, sum_j bf16(out[row(t, j)] * bf16(w[t, j])) in float32, in
    order j; a pair without a row (sentinel) adds zero."""
    out = bf16.from_bits(np.asarray(out_bits)).astype(np.float64)
    rows = np.asarray(row_of_pair).reshape(num_tokens, top_k)
    w = bf16.from_bits(bf16.to_bits(np.asarray(topk_weights, dtype=np.float64))).astype(np.float64)
    w = w.reshape(num_tokens, top_k)
    acc = np.zeros((num_tokens, out.shape[1]), dtype=np.float32)
    for j in range(top_k):
        r = rows[:, j]
        term = np.zeros_like(acc, dtype=np.float64)
        ok = r >= 0
        term[ok] = out[r[ok]] * w[ok, j][:, None]  # exact in float64
        term32 = bf16.from_bits(bf16.to_bits(term)).astype(np.float32)  # bf16 product, exact in float32
        acc = (acc + term32).astype(np.float32)  # one float32 rounding per pair, in order j
    return bf16.to_bits(acc.astype(np.float64))


def expert_mlp_ref(x_rows, w_up, s_up, w_down, s_down):
    """One expert on rows of bf16 values: quantize, up GEMM, SwiGLU, quantize, down GEMM.

    Returns (out_bits [rows, H], proj_bits [rows, 2I], h_bits [rows, I])."""
    q, s = quant.quant_act_ref(np.asarray(x_rows, dtype=np.float32))
    proj = gemm.gemm_ref(q, s, w_up, s_up)
    h = swiglu_ref(proj)
    q2, s2 = quant.quant_act_ref(bf16.from_bits(h).astype(np.float32))
    return gemm.gemm_ref(q2, s2, w_down, s_down), proj, h


def moe_forward_ref(hidden, topk_ids, topk_weights, w_up, s_up, w_down, s_down):
    """The page's FP8 experts forward on bf16 values hidden [T, H]; returns y bf16 bits [T, H].

    Written per pair, without the padded buffer: every (token, expert) pair is one row of its
    expert's MLP (rows are independent), then the pairs are combined per token."""
    hidden = np.asarray(hidden, dtype=np.float32)
    ids = np.asarray(topk_ids).astype(np.int64)
    t, k = ids.shape
    e_count = np.asarray(w_up).shape[0]
    flat = ids.reshape(-1)
    out_rows = np.zeros((t * k, np.asarray(w_down).shape[1]), dtype=np.uint16)
    for e in range(e_count):
        pairs = np.nonzero(flat == e)[0]
        if pairs.size == 0:
            continue
        o, _, _ = expert_mlp_ref(hidden[pairs // k], w_up[e], s_up[e], w_down[e], s_down[e])
        out_rows[pairs] = o
    row_of_pair = np.where((flat >= 0) & (flat < e_count), np.arange(t * k), -1)
    return combine_ref(out_rows, row_of_pair, topk_weights, t, k)
