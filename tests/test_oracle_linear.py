"""Pins of the oracle's FP8 linear layer (CPU): the bias step against torch's own bf16 add and
against exact rationals, and the composition with the pinned quantizer and GEMM."""

from fractions import Fraction

import numpy as np
import torch

from oracle import bf16, gemm, linear, quant
from tests.exact import nearest_bf16, nearest_f32


def _bf16_values(rng, shape, scale_exp):
    """Random bf16 values (float32 array) with magnitudes spread over 2**[-scale_exp, scale_exp]."""
    mant = rng.uniform(-2, 2, shape)
    exps = rng.integers(-scale_exp, scale_exp + 1, shape)
    v = torch.from_numpy((mant * np.exp2(exps)).astype(np.float32)).to(torch.bfloat16)
    return v.float().numpy()


def test_bias_add_equals_torch_bf16_add():
    """The page adds the bias with output.add_(bias) on a bf16 tensor; torch's CPU bf16 add is
    the library routine this step must equal bit for bit (magnitudes spread over 2**+-20, so
    both cancellation and absorption occur)."""
    rng = np.random.default_rng(11)
    c = _bf16_values(rng, (64, 96), 20)
    b = _bf16_values(rng, (96,), 20)
    b[:8] = -c[0, :8]  # exact cancellation to zero
    c_bits = bf16.to_bits(c.astype(np.float64))
    got = linear.bias_add_bf16(c_bits, b)
    want = (torch.from_numpy(c).to(torch.bfloat16) + torch.from_numpy(b).to(torch.bfloat16)).view(torch.int16)
    np.testing.assert_array_equal(got, want.numpy().view(np.uint16))


def test_bias_add_exact_rationals():
    """bf16(float32(c + b)) computed with exact rationals: one float32 rounding of the exact
    sum, then one bf16 rounding (the double rounding of the page's bf16 add)."""
    rng = np.random.default_rng(12)
    c = _bf16_values(rng, (8, 40), 40)
    b = _bf16_values(rng, (40,), 40)
    got = bf16.from_bits(linear.bias_add_bf16(bf16.to_bits(c.astype(np.float64)), b))
    for i in range(c.shape[0]):
        for j in range(c.shape[1]):
            exact = Fraction(float(c[i, j])) + Fraction(float(b[j]))
            assert Fraction(float(got[i, j])) == nearest_bf16(nearest_f32(exact)), (i, j)


def test_linear_without_bias_is_quantize_then_gemm():
    rng = np.random.default_rng(13)
    x = torch.from_numpy(rng.standard_normal((7, 256)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    w_q = rng.integers(0, 0x7E, (136, 256)).astype(np.uint8)
    w_s = rng.uniform(1e-3, 1e-2, (2, 2)).astype(np.float32)
    out, c, q, s = linear.linear_ref(x, w_q, w_s)
    q2, s2 = quant.quant_act_ref(x)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(out, gemm.gemm_ref(q2, s2, w_q, w_s))
    np.testing.assert_array_equal(out, c)


def test_linear_bias_is_added_after_bf16_rounding():
    """A bias equal to -bf16(C) cancels exactly (the bias meets the rounded bf16 output, not the
    float32 accumulator): every output is zero."""
    rng = np.random.default_rng(14)
    x = torch.from_numpy(rng.standard_normal((3, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    w_q = rng.integers(0, 0x7E, (16, 128)).astype(np.uint8)
    w_s = rng.uniform(1e-3, 1e-2, (1, 1)).astype(np.float32)
    _, c, _, _ = linear.linear_ref(x, w_q, w_s)
    row0 = bf16.from_bits(c[0]).astype(np.float32)
    out, _, _, _ = linear.linear_ref(x[:1], w_q, w_s, bias=-row0)
    assert (bf16.from_bits(out) == 0).all()


def test_f16_rounding_against_numpy_and_exact_rationals():
    """fp16 RNE from float64 against numpy's own float64 -> float16 cast (correctly rounded) on
    values spread over every binade incl. subnormals and overflow, and exact rationals on ties."""
    from oracle import f16

    rng = np.random.default_rng(41)
    v = rng.uniform(-1, 1, 400000) * np.exp2(rng.integers(-30, 18, 400000))
    np.testing.assert_array_equal(f16.to_bits(v), v.astype(np.float16).view(np.uint16))
    # ties: halfway between two fp16 neighbours rounds to the even one
    for a in (1.0, 1.0 + 2.0**-10, 2.0**-14, 3 * 2.0**-24):
        mid = Fraction(a) + Fraction(float(f16.ulp(a))) / 2
        got = Fraction(float(f16.round_to_f16(float(mid))))
        lo, hi = Fraction(a), Fraction(a) + Fraction(float(f16.ulp(a)))
        want = lo if (int(np.float16(a).view(np.uint16)) & 1) == 0 else hi
        assert got == want, a
    assert np.isinf(f16.round_to_f16(65520.0)) and f16.round_to_f16(65519.0) == 65504.0


def test_f16_bias_add_equals_torch_f16_add():
    rng = np.random.default_rng(42)
    c = torch.from_numpy(rng.standard_normal((32, 64)) * 100).to(torch.float16)
    b = torch.from_numpy(rng.standard_normal(64) * 3).to(torch.float16)
    got = linear.bias_add_f16(c.view(torch.int16).numpy().view(np.uint16), b.float().numpy())
    np.testing.assert_array_equal(got, (c + b).view(torch.int16).numpy().view(np.uint16))
