"""Pins of the oracle's blockwise GEMM and grouped GEMM (CPU): brute force, special cases, invariants."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16, gemm, quant
from tests.exact import e4m3_values_torch, nearest_bf16

E4 = e4m3_values_torch()  # decoded by torch, independent of oracle.e4m3


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return c


def _rand_case(rng, m, n, k):
    a = _rand_codes(rng, (m, k))
    b = _rand_codes(rng, (n, k))
    a_s = rng.uniform(1e-3, 2.0, (m, -(-k // 128))).astype(np.float32)
    b_s = rng.uniform(1e-3, 1e-2, (-(-n // 128), -(-k // 128))).astype(np.float32)
    return a, a_s, b, b_s


def _brute_force(a, a_s, b, b_s, rows, cols):
    """C[m, n] with exact rationals, rounded once to bf16."""
    k = a.shape[1]
    out = {}
    for m in rows:
        for n in cols:
            total = Fraction(0)
            for kb in range(-(-k // 128)):
                p = sum((E4[a[m, kk]] * E4[b[n, kk]] for kk in range(kb * 128, min(k, kb * 128 + 128))), Fraction(0))
                total += p * Fraction(float(a_s[m, kb])) * Fraction(float(b_s[n // 128, kb]))
            out[(m, n)] = nearest_bf16(total)
    return out


@pytest.mark.parametrize("m,n,k", [(3, 5, 128), (4, 136, 256), (2, 7, 384), (1, 3, 200)])
def test_brute_force_exact_rationals(m, n, k):
    rng = np.random.default_rng(m * 1000 + n + k)
    a, a_s, b, b_s = _rand_case(rng, m, n, k)
    cols = list(range(n)) if n <= 8 else [0, 5, 127, 128, 129, 135]
    got = gemm.gemm_ref(a, a_s, b, b_s, cols=np.array(cols))
    want = _brute_force(a, a_s, b, b_s, range(m), cols)
    for i in range(m):
        for j, n_ in enumerate(cols):
            assert Fraction(float(bf16.from_bits(got[i, j]))) == want[(i, n_)], (i, n_)


def test_unit_scales_k128_is_integer_fp8_dot():
    """With As = Bs = 1 and K = 128, C is the plain FP8 dot product: an integer matmul of 2**9 * values."""
    rng = np.random.default_rng(1)
    a, _, b, _ = _rand_case(rng, 16, 24, 128)
    ones_a = np.ones((16, 1), np.float32)
    ones_b = np.ones((1, 1), np.float32)
    acc, _ = gemm.gemm_acc_ref(a, ones_a, b, ones_b)
    to_int = np.vectorize(lambda c: int(E4[c] * 512))
    ai = to_int(a).astype(np.int64)
    bi = to_int(b).astype(np.int64)
    ref = (ai @ bi.T).astype(np.float64) / 2.0**18
    assert np.array_equal(acc, ref)


def test_constant_scales_closed_form():
    """As = a, Bs = b constant: C = a * b * (A . B^T) (per-tensor scales expanded to blocks)."""
    rng = np.random.default_rng(2)
    a, _, b, _ = _rand_case(rng, 9, 200, 640)
    av, bv = np.float32(0.37), np.float32(0.0041)
    a_s = np.full((9, 5), av, np.float32)
    b_s = np.full((2, 5), bv, np.float32)
    acc, absum = gemm.gemm_acc_ref(a, a_s, b, b_s)
    dec = np.vectorize(lambda c: float(E4[c]))
    full = dec(a) @ dec(b).T  # exact (integers times 2**-18, far below 2**53 units)
    ref = full * (np.float64(av) * np.float64(bv))
    # the oracle rounds each of the 5 block terms and their running sum in float64
    assert (np.abs(acc - ref) <= 10 * 2.0**-53 * absum).all()
    assert np.array_equal(gemm.gemm_ref(a, a_s, b, b_s), bf16.to_bits(ref))


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(3)
    a, a_s, b, b_s = _rand_case(rng, 6, 130, 384)
    acc, _ = gemm.gemm_acc_ref(a, a_s, b, b_s)
    acc2, _ = gemm.gemm_acc_ref(a, a_s * np.float32(8.0), b, b_s * np.float32(0.25))
    assert np.array_equal(acc2, acc * 2.0)


def test_k_block_permutation_invariance():
    rng = np.random.default_rng(4)
    a, a_s, b, b_s = _rand_case(rng, 5, 140, 512)
    perm = np.array([2, 0, 3, 1])
    cols = np.concatenate([np.arange(p * 128, p * 128 + 128) for p in perm])
    acc, _ = gemm.gemm_acc_ref(a, a_s, b, b_s)
    acc_p, absum = gemm.gemm_acc_ref(a[:, cols], a_s[:, perm], b[:, cols], b_s[:, perm])
    assert (np.abs(acc_p - acc) <= 16 * 2.0**-53 * absum).all()


def test_weight_scale_strip_locality():
    """Changing Bs[nb, :] changes only output columns of strip nb (N = 576: strip 4 is 512..575)."""
    a_f, w = workloads.page2_case()
    a_q, a_s = quant.quant_act_ref(a_f[:4].numpy())
    b_q, b_s = w.q.numpy(), w.s.numpy()
    acc, _ = gemm.gemm_acc_ref(a_q, a_s, b_q, b_s)
    for nb in (0, 4):
        b_s2 = b_s.copy()
        b_s2[nb] *= np.float32(3.0)
        acc2, _ = gemm.gemm_acc_ref(a_q, a_s, b_q, b_s2)
        changed = np.any(acc2 != acc, axis=0)
        strip = (np.arange(576) // 128) == nb
        assert np.array_equal(changed, strip)


def test_subset_rows_cols_equal_full():
    rng = np.random.default_rng(6)
    a, a_s, b, b_s = _rand_case(rng, 10, 300, 256)
    full = gemm.gemm_ref(a, a_s, b, b_s)
    rows, cols = np.array([9, 0, 4]), np.array([299, 1, 128, 255])
    assert np.array_equal(gemm.gemm_ref(a, a_s, b, b_s, rows, cols), full[np.ix_(rows, cols)])


def test_shape_checks():
    rng = np.random.default_rng(7)
    a, a_s, b, b_s = _rand_case(rng, 2, 3, 256)
    with pytest.raises(ValueError):
        gemm.gemm_ref(a, a_s[:, :1], b, b_s)
    with pytest.raises(ValueError):
        gemm.gemm_ref(a, a_s, b[:, :128], b_s)


def test_grouped_brute_force_and_padding_rows():
    rng = np.random.default_rng(8)
    g_count, n, k = 3, 6, 256
    layout = np.array([0, 0, -1, 2, 2, 2, -1, 1], dtype=np.int32)
    m = layout.size
    a = _rand_codes(rng, (m, k))
    a_s = rng.uniform(0.1, 1, (m, 2)).astype(np.float32)
    b = np.stack([_rand_codes(rng, (n, k)) for _ in range(g_count)])
    b_s = rng.uniform(1e-3, 1e-2, (g_count, 1, 2)).astype(np.float32)
    rows, bits = gemm.grouped_gemm_contiguous_ref(a, a_s, b, b_s, layout)
    assert rows.tolist() == [0, 1, 3, 4, 5, 7]
    for i, r in enumerate(rows):
        g = layout[r]
        want = _brute_force(a, a_s, b[g], b_s[g], [r], range(n))
        for c in range(n):
            assert Fraction(float(bf16.from_bits(bits[i, c]))) == want[(r, c)]
    # padding rows hold garbage (NaN codes and NaN scales): valid rows are unchanged
    a2, a_s2 = a.copy(), a_s.copy()
    a2[layout < 0] = 0x7F
    a_s2[layout < 0] = np.nan
    rows2, bits2 = gemm.grouped_gemm_contiguous_ref(a2, a_s2, b, b_s, layout)
    assert np.array_equal(rows2, rows) and np.array_equal(bits2, bits)
    with pytest.raises(ValueError):
        gemm.grouped_gemm_contiguous_ref(a, a_s, b, b_s, np.array([0, 3, 0, 0, 0, 0, 0, 0], np.int32))


def test_moe_layout_generator_contract():
    counts = workloads.moe_counts()
    assert counts.sum() == 4096 and counts.size == 16
    layout = workloads.moe_layout(counts)
    assert layout.size % 128 == 0
    blocks = layout.reshape(-1, 128)
    for blk in blocks:
        ids = set(blk[blk >= 0].tolist())
        assert len(ids) <= 1  # every 128-row block belongs to one expert
    for g, c in enumerate(counts):
        assert (layout == g).sum() == c
    assert torch.from_numpy(layout).dtype == torch.int32


def test_grouped_nn_brute_force_and_against_nt():
    """NN expert weights [G, K, N]: exact rationals on a tiny case, and the same numbers as the NT
    form when the NT operand is the transpose (a layout, not a different product)."""
    from fractions import Fraction

    from oracle import e4m3, gemm

    rng = np.random.default_rng(71)
    g_count, m, n, k = 2, 256, 136, 256
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8)
    b_nn = rng.integers(0, 0x7E, (g_count, k, n)).astype(np.uint8) | (rng.integers(0, 2, (g_count, k, n)).astype(np.uint8) << 7)
    a_s = rng.uniform(1e-3, 1e-2, (m, 2)).astype(np.float32)
    bs_nn = rng.uniform(1e-3, 1e-2, (g_count, 2, 2)).astype(np.float32)
    layout = np.concatenate([np.zeros(100, np.int32), -np.ones(28, np.int32), np.ones(128, np.int32)])
    rows, acc = gemm.grouped_gemm_contiguous_nn_acc_ref(a, a_s, b_nn, bs_nn, layout)
    assert rows.tolist() == list(range(100)) + list(range(128, 256))
    av, bv = e4m3.decode(a), e4m3.decode(b_nn)
    for i, r in enumerate(rows[::37]):
        for c in (0, 77, 128, 135):
            g = layout[r]
            want = Fraction(0)
            for kb in range(2):
                s = sum(Fraction(float(av[r, kk])) * Fraction(float(bv[g, kk, c])) for kk in range(kb * 128, kb * 128 + 128))
                want += s * Fraction(float(a_s[r, kb])) * Fraction(float(bs_nn[g, kb, c // 128]))
            assert abs(Fraction(float(acc[i * 37, c])) - want) <= abs(want) * Fraction(1, 2**46), (r, c)  # float64 rounding only
    rows2, acc2, _ = gemm.grouped_gemm_contiguous_acc_ref(a, a_s, b_nn.transpose(0, 2, 1), bs_nn.transpose(0, 2, 1), layout)
    np.testing.assert_array_equal(rows, rows2)
    np.testing.assert_allclose(acc, acc2, rtol=1e-14, atol=0)
