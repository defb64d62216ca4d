"""Pins of the oracle's 1x64 / 128x64 layout (CPU): the quantizer with 64-wide groups and the
blockwise GEMM with 64-wide K scale blocks (weight blocks stay 128 rows tall).

Each pin would catch a plausible slip: a group or block width left at 128, a weight block row
taken as n // 64, the two halves of a 128-wide K range given each other's scales, a partial last
group sized wrong."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, gemm, quant
from tests.exact import e4m3_values_torch, nearest_bf16

E4 = e4m3_values_torch()  # decoded by torch, independent of oracle.e4m3


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return c


def _case(rng, m, n, k):
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    a_s = rng.uniform(1e-3, 2.0, (m, -(-k // 64))).astype(np.float32)
    b_s = rng.uniform(1e-3, 1e-2, (-(-n // 128), -(-k // 64))).astype(np.float32)
    return a, a_s, b, b_s


@pytest.mark.parametrize("k", [448, 400, 64, 16])
def test_quant_64_groups_are_the_pinned_quantizer_on_each_slice(k):
    """Every 64-wide group quantizes as the (pinned) 1x128 quantizer does a matrix holding only
    that group's columns: same codes, same scale; the last group may be shorter."""
    rng = np.random.default_rng(k)
    x = (rng.standard_normal((6, k)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    x[2, :] = 0.0  # an all-zero row: the amax floor
    q, s = quant.quant_act_ref(x, group=64)
    assert q.shape == (6, k) and s.shape == (6, -(-k // 64))
    for g in range(-(-k // 64)):
        cols = slice(64 * g, min(64 * g + 64, k))
        q1, s1 = quant.quant_act_ref(x[:, cols])
        np.testing.assert_array_equal(q[:, cols], q1)
        np.testing.assert_array_equal(s[:, g], s1[:, 0])


def test_quant_64_scale_closed_form():
    """s = fl32(max |x| / 448) per 64 columns: a row whose two halves of 128 columns have amax
    448 * 2^-3 and 448 * 2^5 gets scales 2^-3 and 2^5 (a 128-wide group would give 2^5 to both)."""
    x = np.zeros((1, 128), np.float32)
    x[0, 10] = -448 * 2.0**-3
    x[0, 100] = 448 * 2.0**5
    _, s = quant.quant_act_ref(x, group=64)
    np.testing.assert_array_equal(s[0], np.float32([2.0**-3, 2.0**5]))
    _, s128 = quant.quant_act_ref(x)
    np.testing.assert_array_equal(s128[0], np.float32([2.0**5]))


def _brute(a, a_s, b, b_s, rows, cols):
    k = a.shape[1]
    out = {}
    for m in rows:
        for n in cols:
            total = Fraction(0)
            for g in range(-(-k // 64)):
                p = sum((E4[a[m, kk]] * E4[b[n, kk]] for kk in range(64 * g, min(k, 64 * g + 64))), Fraction(0))
                total += p * Fraction(float(a_s[m, g])) * Fraction(float(b_s[n // 128, g]))
            out[(m, n)] = nearest_bf16(total)
    return out


@pytest.mark.parametrize("m,n,k", [(2, 5, 128), (3, 136, 208), (1, 130, 64), (2, 3, 16)])
def test_gemm_64_brute_force_exact_rationals(m, n, k):
    rng = np.random.default_rng(m * 7 + n + k)
    a, a_s, b, b_s = _case(rng, m, n, k)
    cols = list(range(n)) if n <= 8 else [0, 64, 127, 128, 129, n - 1]
    got = gemm.gemm_ref(a, a_s, b, b_s, cols=np.array(cols), k_block=64)
    want = _brute(a, a_s, b, b_s, range(m), cols)
    for i in range(m):
        for j, n_ in enumerate(cols):
            assert Fraction(float(bf16.from_bits(got[i, j]))) == want[(i, n_)], (i, n_)


def test_gemm_64_with_equal_half_scales_is_the_128_product():
    """Scales equal on both 64-halves of every 128 columns: the 1x64 product equals the pinned
    1x128 one (up to float64 rounding of the order of the sum)."""
    rng = np.random.default_rng(5)
    a, a_s, b, b_s = _case(rng, 7, 300, 512)
    a_s[:, 1::2] = a_s[:, 0::2]
    b_s[:, 1::2] = b_s[:, 0::2]
    acc64, _ = gemm.gemm_acc_ref(a, a_s, b, b_s, k_block=64)
    acc128, absum = gemm.gemm_acc_ref(a, a_s[:, 0::2], b, b_s[:, 0::2])
    # 8 blocks of 128: at most ~16 float64 roundings of terms no larger than absum
    assert (np.abs(acc64 - acc128) <= 2.0**-46 * absum).all()


def test_gemm_64_swapping_half_scales_changes_the_result():
    rng = np.random.default_rng(6)
    a, a_s, b, b_s = _case(rng, 4, 200, 256)
    acc, _ = gemm.gemm_acc_ref(a, a_s, b, b_s, k_block=64)
    a_sw = a_s.copy()
    a_sw[:, [0, 1]] = a_sw[:, [1, 0]]
    acc_sw, _ = gemm.gemm_acc_ref(a, a_sw, b, b_s, k_block=64)
    assert np.abs(acc - acc_sw).max() > 1e-3 * np.abs(acc).max()


def test_gemm_64_weight_blocks_are_128_rows_tall():
    """Changing the scale of weight block row 1 (rows 128..255) changes exactly those columns."""
    rng = np.random.default_rng(7)
    a, a_s, b, b_s = _case(rng, 3, 300, 192)
    acc, _ = gemm.gemm_acc_ref(a, a_s, b, b_s, k_block=64)
    b2 = b_s.copy()
    b2[1] *= 2
    acc2, _ = gemm.gemm_acc_ref(a, a_s, b, b2, k_block=64)
    changed = np.nonzero(np.abs(acc2 - acc).max(axis=0) > 0)[0]
    assert changed.min() >= 128 and changed.max() <= 255


def test_gemm_64_unit_scales_is_the_plain_fp8_dot():
    rng = np.random.default_rng(8)
    a, _, b, _ = _case(rng, 5, 9, 320)
    acc, _ = gemm.gemm_acc_ref(a, np.ones((5, 5), np.float32), b, np.ones((1, 5), np.float32), k_block=64)
    av = np.vectorize(lambda c: float(E4[c]))(a)
    bv = np.vectorize(lambda c: float(E4[c]))(b)
    np.testing.assert_array_equal(acc, av @ bv.T)  # each partial sum exact in float64


def test_gemm_64_shape_checks():
    a = np.zeros((2, 192), np.uint8)
    b = np.zeros((3, 192), np.uint8)
    with pytest.raises(ValueError):
        gemm.gemm_acc_ref(a, np.ones((2, 2), np.float32), b, np.ones((1, 3), np.float32), k_block=64)
    with pytest.raises(ValueError):
        gemm.gemm_acc_ref(a, np.ones((2, 3), np.float32), b, np.ones((1, 2), np.float32), k_block=64)
    with pytest.raises(ValueError):
        gemm.gemm_acc_ref(a, np.ones((2, 3), np.float32), b, np.ones((1, 3), np.float32), k_block=32)
    gemm.gemm_acc_ref(a, np.ones((2, 3), np.float32), b, np.ones((1, 3), np.float32), k_block=64)
