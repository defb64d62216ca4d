"""Pins of the oracle's MoE chain (CPU): the contiguous layout against the page's sort-based
construction and a hand-worked example, SwiGLU against torch's own float64 silu, the combine on
exact sums and NaN sentinel rows, and the chain against a single-expert dense MLP."""

import numpy as np
import torch

from oracle import bf16, gemm, moe, quant
import workloads


def test_layout_hand_example():
    """ids [1, 0, 1, 2] with E = 2 (id 2 is a sentinel), alignment 4: counts [1, 2] -> blocks of
    4 rows at 0 and 4; pairs 1 -> row 0, 0 -> row 4, 2 -> row 5; the buffer has 4 + 2 * 3 rows."""
    rows, pairs, layout, start = moe.layout_ref(np.array([1, 0, 1, 2]), 2, 4)
    assert rows.tolist() == [4, 0, 5, -1]
    assert start.tolist() == [0, 4, 8]
    assert layout.tolist() == [0, -1, -1, -1, 1, 1, -1, -1, -1, -1]
    assert pairs.tolist() == [1, -1, -1, -1, 0, 2, -1, -1, -1, -1]


def _page_construction(ids: torch.Tensor, e: int, align: int):
    """The page's steps with torch: sort by expert (stable here), histc counts, aligned counts,
    exclusive cumsum of the padding, sorted_to_padded = arange + cumulative_padding[sorted id]."""
    ids_sorted, perm = torch.sort(ids, stable=True)
    counts = torch.histc(ids_sorted.float(), bins=e, min=0, max=e - 1).long()
    aligned = (counts + align - 1) // align * align
    cum_pad = torch.nn.functional.pad((aligned - counts).cumsum(0), (1, 0))
    sorted_to_padded = torch.arange(ids.numel()) + cum_pad[ids_sorted]
    row_of_pair = torch.empty_like(sorted_to_padded)
    row_of_pair[perm] = sorted_to_padded
    return row_of_pair, ids.numel() + min(ids.numel(), e) * (align - 1)


def test_layout_matches_page_construction():
    for seed, (s, e, align) in enumerate([(4096, 16, 128), (1000, 7, 32), (64, 128, 128), (300, 3, 1)]):
        rng = np.random.default_rng(seed)
        ids = rng.integers(0, e + 1, s)  # includes sentinels == E
        rows, pairs, layout, start = moe.layout_ref(ids, e, align)
        want, m_pad = _page_construction(torch.from_numpy(ids), e, align)
        valid = ids < e
        np.testing.assert_array_equal(rows[valid], want.numpy()[valid])
        assert (rows[~valid] == -1).all()
        assert layout.size == m_pad and pairs.size == m_pad
        # invariants: aligned blocks in expert order, pairs in index order inside each block
        assert (start[:-1] % align == 0).all() and start[-1] <= m_pad
        for x in range(e):
            r = np.nonzero(layout == x)[0]
            assert r.size == 0 or (r[0] == start[x] and np.all(np.diff(r) == 1))
            assert np.all(np.diff(pairs[r]) > 0) and np.all(ids[pairs[r]] == x)
        assert np.all(layout[pairs < 0] == -1)


def test_silu_matches_torch_float64_for_every_bf16():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bf16.from_bits(bits)
    finite = np.isfinite(vals)
    want = torch.nn.functional.silu(torch.from_numpy(vals[finite].astype(np.float64))).to(torch.bfloat16)
    got = moe.silu_bf16_bits(bits[finite])
    np.testing.assert_array_equal(got, want.view(torch.int16).numpy().view(np.uint16))


def test_swiglu_matches_torch_steps():
    rng = np.random.default_rng(3)
    proj = torch.from_numpy(rng.standard_normal((17, 512)).astype(np.float32) * 3).to(torch.bfloat16)
    gate, up = proj[:, :256].double(), proj[:, 256:].double()
    want = (torch.nn.functional.silu(gate).to(torch.bfloat16).double() * up).to(torch.bfloat16)
    got = moe.swiglu_ref(proj.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(got, want.view(torch.int16).numpy().view(np.uint16))
    # silu(x) - silu(-x) = x (exactly, in float64 before rounding)
    x = np.linspace(-20, 20, 4001)
    np.testing.assert_allclose(x / (1 + np.exp(-x)) - (-x) / (1 + np.exp(x)), x, rtol=0, atol=1e-12)


def test_combine_exact_sums_and_nan_sentinels():
    """Out rows of small integers and weights that are powers of two: every product and partial
    sum is exact, so the result is the weighted sum rounded once to bf16. A sentinel pair's row
    holds NaN and must add zero."""
    rng = np.random.default_rng(4)
    t, k, h = 6, 4, 64
    out = rng.integers(-50, 50, (t * k + 3, h)).astype(np.float64)
    w = np.exp2(rng.integers(-3, 2, (t, k))).astype(np.float32)
    rows = rng.permutation(t * k + 3)[: t * k]
    rows[5] = -1  # sentinel pair
    out_bits = bf16.to_bits(out)
    nan_row = np.setdiff1d(np.arange(t * k + 3), rows)[0]
    out_bits[nan_row] = 0x7FC0  # NaN, as allocator reuse may leave there
    y = bf16.from_bits(moe.combine_ref(out_bits, rows, w, t, k))
    want = np.zeros((t, h))
    for p in range(t * k):
        if rows[p] >= 0:
            want[p // k] += out[rows[p]] * w.reshape(-1)[p]
    np.testing.assert_array_equal(y, bf16.from_bits(bf16.to_bits(want)))
    assert np.isfinite(y).all()


def test_chain_with_one_expert_is_the_dense_mlp():
    """top_k = 1, every token on expert 0 with weight 1: the chain is quantize, up GEMM, SwiGLU,
    quantize, down GEMM, and the combine returns that output unchanged."""
    rng = np.random.default_rng(5)
    t, h, i = 9, 256, 128
    x = torch.from_numpy(rng.standard_normal((t, h)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    wu, wd = workloads.weight(2 * i, h, seed=6), workloads.weight(h, i, seed=7)
    ids = np.zeros((t, 1), dtype=np.int64)
    w = np.ones((t, 1), dtype=np.float32)
    y = moe.moe_forward_ref(x, ids, w, wu.q.numpy()[None], wu.s.numpy()[None], wd.q.numpy()[None], wd.s.numpy()[None])
    q, s = quant.quant_act_ref(x)
    proj = gemm.gemm_ref(q, s, wu.q.numpy(), wu.s.numpy())
    hb = moe.swiglu_ref(proj)
    q2, s2 = quant.quant_act_ref(bf16.from_bits(hb).astype(np.float32))
    np.testing.assert_array_equal(y, gemm.gemm_ref(q2, s2, wd.q.numpy(), wd.s.numpy()))


def test_chain_through_padded_buffer_equals_per_pair_form():
    """The page's order of steps (layout, rows of the padded buffer per expert, combine through
    row_of_pair) gives the same bits as the per-pair form; token order is equivariant."""
    rng = np.random.default_rng(8)
    t, k, e, h, i = 11, 3, 4, 128, 128
    x = torch.from_numpy(rng.standard_normal((t, h)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ids = np.stack([rng.choice(e + 1, k, replace=False) for _ in range(t)])  # id e = sentinel
    w = rng.uniform(0, 1, (t, k)).astype(np.float32)
    wu = [workloads.weight(2 * i, h, seed=20 + g) for g in range(e)]
    wd = [workloads.weight(h, i, seed=30 + g) for g in range(e)]
    args = (np.stack([a.q.numpy() for a in wu]), np.stack([a.s.numpy() for a in wu]),
            np.stack([a.q.numpy() for a in wd]), np.stack([a.s.numpy() for a in wd]))
    y = moe.moe_forward_ref(x, ids, w, *args)
    rows, pairs, layout, start = moe.layout_ref(ids, e, 128)
    out = np.zeros((layout.size, h), dtype=np.uint16)
    for g in range(e):
        r = np.nonzero(layout == g)[0]
        if r.size:
            out[r] = moe.expert_mlp_ref(x[pairs[r] // k], args[0][g], args[1][g], args[2][g], args[3][g])[0]
    np.testing.assert_array_equal(moe.combine_ref(out, rows, w, t, k), y)
    perm = rng.permutation(t)
    np.testing.assert_array_equal(moe.moe_forward_ref(x[perm], ids[perm], w[perm], *args), y[perm])
