"""Pins of the oracle's e4m3fn and bf16 codecs against library routines and brute force (CPU)."""

from fractions import Fraction
import os

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3
from tests.exact import nearest_bf16, nearest_e4m3_code

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3.decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # signed zeros too
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_decode_format_landmarks():
    # the page prints finfo(float8_e4m3fn).max = 448: the largest finite code is 0x7E
    assert e4m3.decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert np.isnan(e4m3.decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert e4m3.decode(np.array([0x01], np.uint8))[0] == 2.0**-9  # smallest subnormal
    assert e4m3.decode(np.array([0x08], np.uint8))[0] == 2.0**-6  # smallest normal


def _golden_spot_values():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_spot_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                x, code = line.split()
                rows.append((float.fromhex(x), int(code, 16)))
    return rows


def test_encode_spot_values_fixture():
    rows = _golden_spot_values()
    assert len(rows) >= 10
    xs = np.array([r[0] for r in rows], dtype=np.float64)
    codes = np.array([r[1] for r in rows], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(xs), codes)


def _torch_encode(y32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(y32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _interesting_f32():
    """Every e4m3 value, every midpoint between neighbours, and +-1..3 float32 ulps around each."""
    pos = np.sort(e4m3.decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids]).astype(np.float32)
    around = [base]
    up, dn = base, base
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        around += [up, dn]
    v = np.concatenate(around)
    v = v[(v >= 0) & (v <= 448)]
    return np.concatenate([v, -v]).astype(np.float32)


def test_encode_matches_torch_at_every_rounding_boundary():
    y = _interesting_f32()
    assert np.array_equal(e4m3.encode(y), _torch_encode(y))


def test_encode_matches_torch_strided_all_float32():
    # every 97th float32 bit pattern with |y| <= 448 (and its negation)
    limit = np.array([448.0], np.float32).view(np.uint32)[0]
    for start in range(0, int(limit) + 1, 4_000_000 * 97):
        bits = np.arange(start, min(start + 4_000_000 * 97, int(limit) + 1), 97, dtype=np.uint32)
        y = bits.view(np.float32)
        for v in (y, -y):
            assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_brute_force_enumeration():
    rng = np.random.default_rng(7)
    ys = np.concatenate([rng.uniform(-448, 448, 300), rng.uniform(-0.02, 0.02, 200)]).astype(np.float32)
    got = e4m3.encode(ys)
    for y, c in zip(ys.tolist(), got.tolist()):
        assert c == nearest_e4m3_code(Fraction(y), negative=np.signbit(y))


def test_encode_keeps_sign_of_zero_and_rejects_out_of_range():
    assert e4m3.encode(np.array([-0.0]))[0] == 0x80
    assert e4m3.encode(np.array([-(2.0**-12)]))[0] == 0x80
    assert e4m3.encode(np.array([0.0]))[0] == 0x00
    with pytest.raises(ValueError):
        e4m3.encode(np.array([449.0]))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan]))


def test_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.to_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rounds_float64_once():
    # x = 1 + 2**-8 is a bf16 tie (rounds to even 1.0); one float64 ulp above it must round up,
    # which a detour through float32 would lose.
    cases = [1 + 2.0**-8, 1 + 2.0**-8 + 2.0**-40, 1 + 3 * 2.0**-8, -(1 + 2.0**-8 + 2.0**-40), 2.0**-130 * 1.5]
    rng = np.random.default_rng(3)
    cases += list(rng.normal(0, 1e3, 200)) + list(rng.normal(0, 1e-36, 50))
    for x in cases:
        want = nearest_bf16(Fraction(x))
        got = bf16.round_to_bf16(np.array([x]))[0]
        assert Fraction(got) == want, x
    assert bf16.round_to_bf16(np.array([1 + 2.0**-8 + 2.0**-40]))[0] == 1 + 2.0**-7


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    vals = bf16.from_bits(bits)
    fin = np.isfinite(vals)
    # every finite pattern (including -0.0 = 0x8000 and subnormals) round-trips exactly
    back = bf16.to_bits(vals[fin])
    assert np.array_equal(back, bits[fin])
