"""Pins of the oracle's scale expansion (CPU): the per-token / per-tensor FP8 product against
exact rationals, and the block GEMM on the expanded grids against it."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, gemm, scales
from tests.exact import e4m3_values_torch, nearest_bf16

E4 = e4m3_values_torch()  # decoded by torch, independent of oracle.e4m3


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return c


@pytest.mark.parametrize("m,n,k", [(3, 4, 128), (2, 5, 200), (4, 3, 384)])
def test_per_token_product_exact_rationals(m, n, k):
    rng = np.random.default_rng(m * 100 + k)
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    s_a = rng.uniform(1e-3, 2.0, m).astype(np.float32)
    s_b = np.float32(rng.uniform(1e-4, 1e-2))
    got = scales.gemm_per_token_ref(a, s_a, b, s_b)
    for i in range(m):
        for j in range(n):
            dot = sum((E4[a[i, kk]] * E4[b[j, kk]] for kk in range(k)), Fraction(0))
            want = nearest_bf16(dot * Fraction(float(s_a[i])) * Fraction(float(s_b)))
            assert Fraction(float(bf16.from_bits(got[i, j]))) == want, (i, j)


def test_expanded_grids_shapes_and_values():
    a = scales.expand_act_scales_ref(np.float32(0.5), 5, 300)
    assert a.shape == (5, 3) and (a == np.float32(0.5)).all()
    s = np.arange(1, 6, dtype=np.float32)
    a = scales.expand_act_scales_ref(s, 5, 256)
    assert a.shape == (5, 2) and (a == s[:, None]).all()
    w = scales.expand_weight_scale_ref(np.float32(0.25), 300, 130)
    assert w.shape == (3, 2) and (w == np.float32(0.25)).all()


@pytest.mark.parametrize("per_token", [True, False])
def test_block_gemm_on_expanded_grids_is_the_per_token_product(per_token):
    """The block definition with constant-per-block scales reduces to the per-token product
    (equal bits on this seeded case: the two float64 evaluations differ far below bf16)."""
    rng = np.random.default_rng(7 + per_token)
    m, n, k = 9, 200, 640
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    s_a = rng.uniform(1e-3, 2.0, m).astype(np.float32) if per_token else np.float32(0.75)
    s_b = np.float32(3e-3)
    block = gemm.gemm_ref(a, scales.expand_act_scales_ref(s_a, m, k), b, scales.expand_weight_scale_ref(s_b, n, k))
    np.testing.assert_array_equal(block, scales.gemm_per_token_ref(a, s_a, b, s_b))
