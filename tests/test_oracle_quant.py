"""Pins of the oracle's per-token-group quantizer (CPU): exact-rational brute force, bounds, invariants."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import e4m3, quant
from tests.exact import nearest_e4m3_code, nearest_f32


def _brute_force_group(xg: np.ndarray):
    """Quantize one group with exact rationals: scale and quotient rounded to float32 by enumeration."""
    amax = max(abs(Fraction(float(v))) for v in xg)
    floor = Fraction(float(np.float32(1e-10)))
    s = nearest_f32(max(amax, floor) / 448)
    codes = []
    for v in xg.tolist():
        y = nearest_f32(Fraction(v) / s)
        y = min(max(y, Fraction(-448)), Fraction(448))
        codes.append(nearest_e4m3_code(y, negative=(v < 0 or (v == 0 and np.signbit(v)))))
    return s, codes


def test_brute_force_small_rows():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.uniform(-448, 448, (2, 256)),
        rng.normal(0, 1, (2, 256)),
        rng.normal(0, 1e-3, (1, 256)) * rng.integers(0, 2, (1, 256)),
    ]).astype(np.float32)
    q, s = quant.quant_act_ref(x)
    for m in range(x.shape[0]):
        for g in range(2):
            s_bf, codes_bf = _brute_force_group(x[m, 128 * g:128 * (g + 1)])
            assert Fraction(float(s[m, g])) == s_bf
            assert q[m, 128 * g:128 * (g + 1)].tolist() == codes_bf


def near_tie_rows(n_rows: int = 4, seed: int = 13) -> np.ndarray:
    """Rows whose quotients x/s fall within a few float32 ulps of e4m3 rounding midpoints.

    Column 0 of each 128-group holds the group's amax (a random value, so s = amax/448 is
    not a power of two and 1/s is inexact); the other columns are fl32(mid * s) and its
    float32 neighbours for e4m3 midpoints `mid`. Dividing versus multiplying by 1/s differs
    in the last float32 bit for some of these, which moves the e4m3 rounding.
    """
    rng = np.random.default_rng(seed)
    pos = np.sort(e4m3.decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    rows = []
    for _ in range(n_rows):
        row = []
        for _g in range(2):
            amax = np.float32(rng.uniform(100, 448))
            s = amax / np.float32(448)
            picks = rng.choice(mids[mids < 440], 26, replace=False)
            vals = []
            for mid in picks:
                c = np.float32(np.float64(mid) * np.float64(s))
                vals += [np.nextafter(np.nextafter(c, np.float32(-1e9)), np.float32(-1e9)),
                         np.nextafter(c, np.float32(-1e9)), c, np.nextafter(c, np.float32(1e9)),
                         np.nextafter(np.nextafter(c, np.float32(1e9)), np.float32(1e9))]
            vals = np.array(vals[:127], dtype=np.float32)
            vals *= np.where(rng.random(127) < 0.5, -1, 1).astype(np.float32)
            row.append(np.concatenate([[amax], vals]).astype(np.float32))
        rows.append(np.concatenate(row))
    return np.stack(rows)


def test_brute_force_near_e4m3_ties():
    x = near_tie_rows()
    q, s = quant.quant_act_ref(x)
    for m in range(x.shape[0]):
        for g in range(2):
            s_bf, codes_bf = _brute_force_group(x[m, 128 * g:128 * (g + 1)])
            assert Fraction(float(s[m, g])) == s_bf
            assert q[m, 128 * g:128 * (g + 1)].tolist() == codes_bf


def test_round_trip_bound_and_argmax_code():
    a, _ = workloads.page2_case()
    x = a.numpy()
    q, s = quant.quant_act_ref(x)
    assert q.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (83, 56)
    recon = quant.dequant_ref(q, s)
    s_full = np.repeat(s.astype(np.float64), 128, axis=1)
    bound = s_full * e4m3.ulp(q) / 2 + 2.0**-23 * np.abs(x)
    assert (np.abs(x - recon) <= bound).all()
    # the largest-magnitude element of every group maps to +-448 (code 0x7E / 0xFE)
    xg = x.reshape(83, 56, 128)
    qg = q.reshape(83, 56, 128)
    arg = np.abs(xg).argmax(axis=2)
    picked = np.take_along_axis(qg, arg[..., None], axis=2)[..., 0]
    assert np.isin(picked, [0x7E, 0xFE]).all()
    # scale is amax / 448 to within one float32 rounding
    amax = np.abs(xg).max(axis=2).astype(np.float64)
    assert np.allclose(s.astype(np.float64), amax / 448, rtol=2.0**-24, atol=0)


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 3, (4, 384)).astype(np.float32)
    q, s = quant.quant_act_ref(x)
    for j in (-7, 3, 20):
        q2, s2 = quant.quant_act_ref(x * np.float32(2.0**j))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0**j))


def test_zero_group_and_partial_last_group():
    x = np.zeros((3, 300), dtype=np.float32)
    x[1, 200:] = np.linspace(-5, 5, 100, dtype=np.float32)
    x[2, 5] = -0.0
    q, s = quant.quant_act_ref(x)
    assert s.shape == (3, 3)
    assert np.all(s[0] == np.float32(1e-10) / np.float32(448))
    assert np.all(q[0] == 0)
    assert q[2, 5] == 0x80  # negative zero keeps its sign
    # group 2 has 44 columns: its amax is taken over those only
    assert s[1, 2] == np.float32(5.0) / np.float32(448)
    assert s[1, 1] == np.float32(np.abs(x[1, 128:256]).max()) / np.float32(448)


def test_bf16_input_equals_its_float32_widening():
    xb = workloads.act_normal_bf16(8, 512, seed=1)
    q1, s1 = quant.quant_act_ref(xb.float().numpy())
    # through a numpy float32 view of the same values
    q2, s2 = quant.quant_act_ref(xb.to(torch.float32).numpy().astype(np.float32))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_rejects_non_2d():
    with pytest.raises(ValueError):
        quant.quant_act_ref(np.zeros(10, np.float32))
