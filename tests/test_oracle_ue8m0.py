"""Pins of the oracle's UE8M0 scale factors and power-of-two quantizer (CPU): torch's own
float8_e8m0fnu conversions, closed forms with exact rationals, brute force and invariants."""

import math
from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3, quant, ue8m0
from tests.exact import nearest_e4m3_code, nearest_f32


def _positive_normals(rng, n):
    bits = rng.integers(0x00800000, 0x7F000000, n, dtype=np.uint32)  # below 2**127, so the ceiling stays finite
    return bits.view(np.float32)


def test_powers_of_two_round_trip_through_torch_e8m0():
    """Every power of two 2**-127 .. 2**127 is a fixed point of the ceiling, and torch's own
    float32 <-> float8_e8m0fnu conversions agree with the codec on it."""
    p = np.ldexp(np.float32(1), np.arange(-127, 128)).astype(np.float32)
    np.testing.assert_array_equal(ue8m0.ceil_to_ue8m0(p[1:]), p[1:])
    t = torch.from_numpy(p).to(torch.float8_e8m0fnu)
    np.testing.assert_array_equal(ue8m0.encode(p), t.view(torch.uint8).numpy())
    np.testing.assert_array_equal(ue8m0.decode(ue8m0.encode(p)), t.float().numpy().astype(np.float64))


def test_ceil_closed_form():
    """ceil_to_ue8m0(v) = 2**ceil(log2 v), exactly, checked with frexp on exact rationals."""
    rng = np.random.default_rng(22)
    v = _positive_normals(rng, 5000)
    got = ue8m0.ceil_to_ue8m0(v)
    for a, b in zip(v.tolist(), got.tolist()):
        mant, ex = math.frexp(a)  # a = mant * 2**ex, mant in [0.5, 1)
        want = Fraction(2) ** (ex - 1) if mant == 0.5 else Fraction(2) ** ex
        assert Fraction(b) == want, (a, b)


def test_codec_matches_torch_for_every_byte():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    got = ue8m0.decode(codes)
    np.testing.assert_array_equal(got[:255], want[:255])
    assert np.isnan(got[255]) and np.isnan(want[255])
    np.testing.assert_array_equal(ue8m0.encode(got[:255].astype(np.float32)), codes[:255])


def _brute_force_group(xg):
    amax = max(abs(Fraction(float(v))) for v in xg)
    s32 = nearest_f32(max(amax, Fraction(float(np.float32(1e-10)))) / 448)
    s = Fraction(1)
    while s < s32:
        s *= 2
    while s / 2 >= s32:
        s /= 2
    codes = []
    for v in xg.tolist():
        y = min(max(Fraction(v) / s, Fraction(-448)), Fraction(448))  # exact quotient: s is a power of two
        codes.append(nearest_e4m3_code(y, negative=(v < 0 or (v == 0 and np.signbit(v)))))
    return s, codes


def test_brute_force_small_rows():
    rng = np.random.default_rng(23)
    x = np.concatenate([
        rng.uniform(-448, 448, (2, 256)),
        rng.standard_normal((2, 256)) * 1e-3,
        np.ldexp(rng.uniform(-1, 1, (2, 256)), rng.integers(-30, 30, (2, 256))),
    ]).astype(np.float32)
    x[0, 5] = 448.0 * 2.0**-3  # a group whose amax / 448 is a power of two
    q, e = ue8m0.quant_act_ue8m0_ref(x)
    for m in range(x.shape[0]):
        for g in range(2):
            s, codes = _brute_force_group(x[m, g * 128:(g + 1) * 128])
            assert Fraction(float(ue8m0.decode(e[m:m + 1, g])[0])) == s, (m, g)
            assert q[m, g * 128:(g + 1) * 128].tolist() == codes, (m, g)


def test_scale_bounds_and_top_code():
    """s is the smallest power of two >= fl32(amax / 448), so the group's largest element
    lands in (224, 448] and its code is at least 224 in magnitude."""
    rng = np.random.default_rng(24)
    x = (rng.uniform(-1, 1, (64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    q, e = ue8m0.quant_act_ue8m0_ref(x)
    s = ue8m0.decode(e)
    _, s32 = quant.quant_act_ref(x)
    assert np.all(s >= s32) and np.all(s < 2 * s32.astype(np.float64))
    top = np.abs(e4m3.decode(q)).reshape(64, 4, 128).max(axis=2)
    assert np.all(top >= 224) and np.all(top <= 448)
    # round trip: |x - q s| <= s * ulp(q) / 2, i.e. at most half an e4m3 step at the code's binade
    deq = e4m3.decode(q) * np.repeat(s, 128, axis=1)
    step = np.repeat(s, 128, axis=1) * np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(e4m3.decode(q)), 2.0**-6))) - 3), 2.0**-9)
    assert np.all(np.abs(x - deq) <= step / 2 + 1e-30)


def test_equals_float_scale_quantizer_when_the_scale_is_a_power_of_two():
    rng = np.random.default_rng(25)
    x = rng.uniform(-1, 1, (8, 256)).astype(np.float32)
    for m in range(8):
        for g in range(2):
            j = int(rng.integers(0, 128))
            x[m, g * 128:(g + 1) * 128] *= 0.999
            x[m, g * 128 + j] = 448.0 * 2.0 ** (m - 4)  # amax / 448 = 2**(m-4) exactly
    q8, e = ue8m0.quant_act_ue8m0_ref(x)
    qf, sf = quant.quant_act_ref(x)
    np.testing.assert_array_equal(q8, qf)
    np.testing.assert_array_equal(ue8m0.decode(e), sf.astype(np.float64))


def test_power_of_two_scaling_and_zero_group():
    rng = np.random.default_rng(26)
    x = rng.standard_normal((4, 384)).astype(np.float32)
    x[1, 128:256] = 0.0
    q, e = ue8m0.quant_act_ue8m0_ref(x)
    q2, e2 = ue8m0.quant_act_ue8m0_ref(x * np.float32(2.0**9))
    np.testing.assert_array_equal(q, q2)
    nonzero = np.ones_like(e, dtype=bool)
    nonzero[1, 1] = False  # the all-zero group keeps the floor's scale
    np.testing.assert_array_equal(e2.astype(int)[nonzero], e.astype(int)[nonzero] + 9)
    assert e2[1, 1] == e[1, 1]
    assert (q[1, 128:256] == 0).all()
    assert e[1, 1] == ue8m0.encode(ue8m0.ceil_to_ue8m0(np.float32(1e-10) / np.float32(448)))


def test_gemm_with_ue8m0_scales_brute_force():
    """C from UE8M0 codes, with exact rationals, including extreme scale bytes."""
    rng = np.random.default_rng(27)
    a = rng.integers(0, 0x7E, (3, 256)).astype(np.uint8) | (rng.integers(0, 2, (3, 256)).astype(np.uint8) << 7)
    b = rng.integers(0, 0x7E, (136, 256)).astype(np.uint8)
    ae = rng.integers(100, 150, (3, 2)).astype(np.uint8)
    be = rng.integers(100, 150, (2, 2)).astype(np.uint8)
    ae[0, 0], be[1, 1] = 1, 253
    acc, _ = ue8m0.gemm_acc_ue8m0_ref(a, ae, b, be)
    av, bv = e4m3.decode(a), e4m3.decode(b)
    for m in range(3):
        for n in (0, 5, 127, 128, 135):
            want = Fraction(0)
            for kb in range(2):
                p = sum(Fraction(float(av[m, k])) * Fraction(float(bv[n, k])) for k in range(kb * 128, kb * 128 + 128))
                want += p * Fraction(2) ** (int(ae[m, kb]) - 127) * Fraction(2) ** (int(be[n // 128, kb]) - 127)
            # each term is exact in float64; their sum is rounded once (the scales differ by up to 2**150)
            assert float(acc[m, n]) == float(want), (m, n)
