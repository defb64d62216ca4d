"""Pins of the oracle's spacing helpers bf16.ulp, e4m3.ulp and f16.ulp.

These set the per-element acceptance bound of every GEMM parity test (2 ulp of the output format)
and the quantizer's round-trip bound (half an e4m3 step), so each is checked against the spacing
to the next representable value as the library's own decoders give it: torch's bfloat16 and
float8_e4m3fn views of consecutive bit patterns, and numpy's nextafter on float16. An exponent
off by one (a doubled or halved bound) fails at every pattern.
"""

import numpy as np
import torch

from oracle import bf16, e4m3, f16


def _bf16_values(patterns: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(patterns.astype(np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_ulp_is_the_spacing_to_the_next_pattern():
    p = np.arange(0, 0x7F7F, dtype=np.int64)  # every finite non-negative bf16 below the largest
    v, nxt = _bf16_values(p), _bf16_values(p + 1)
    np.testing.assert_array_equal(bf16.ulp(v), nxt - v)
    np.testing.assert_array_equal(bf16.ulp(-v), nxt - v)
    top = _bf16_values(np.array([0x7F7E, 0x7F7F]))  # the largest finite value: same binade below it
    assert bf16.ulp(top[1:]) == top[1] - top[0]
    assert bf16.ulp(np.array([0.0]))[0] == 2.0**-133


def test_bf16_ulp_between_neighbours():
    """A value strictly between two consecutive bf16 values has their distance as its spacing."""
    rng = np.random.default_rng(0)
    p = rng.integers(0, 0x7F7F, 200_000)
    lo, hi = _bf16_values(p), _bf16_values(p + 1)
    x = lo + rng.random(p.size) * (hi - lo)
    keep = (x > lo) & (x < hi)
    np.testing.assert_array_equal(bf16.ulp(x[keep]), (hi - lo)[keep])


def test_e4m3_ulp_is_the_spacing_to_the_next_code():
    codes = np.arange(0, 0x7E, dtype=np.uint8)  # every finite non-negative code below 448
    dec = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(e4m3.ulp(codes), dec[codes.astype(int) + 1] - dec[codes.astype(int)])
    np.testing.assert_array_equal(e4m3.ulp(codes | 0x80), dec[codes.astype(int) + 1] - dec[codes.astype(int)])
    # 448 = 0x7E is not a power of two: its spacing is the one below it in its binade
    assert e4m3.ulp(np.array([0x7E, 0xFE], np.uint8)).tolist() == [dec[0x7E] - dec[0x7D]] * 2 == [32.0, 32.0]
    # the subnormal spacing is 2**-9 and the smallest normal binade shares it
    assert e4m3.ulp(np.array([0x00, 0x07, 0x08], np.uint8)).tolist() == [2.0**-9] * 3


def test_f16_ulp_is_the_spacing_to_the_next_value():
    p = np.arange(0, 0x7BFF, dtype=np.uint16)  # every finite non-negative fp16 below 65504
    v16 = p.view(np.float16)
    v = v16.astype(np.float64)
    nxt = np.nextafter(v16, np.float16(np.inf)).astype(np.float64)
    np.testing.assert_array_equal(f16.ulp(v), nxt - v)
    np.testing.assert_array_equal(f16.ulp(-v), nxt - v)
    top = np.float16(65504.0)
    assert f16.ulp(np.array([65504.0]))[0] == float(top) - float(np.nextafter(top, np.float16(0)))
    rng = np.random.default_rng(1)
    q = rng.integers(0, 0x7BFF, 100_000).astype(np.uint16).view(np.float16)
    lo, hi = q.astype(np.float64), np.nextafter(q, np.float16(np.inf)).astype(np.float64)
    x = lo + rng.random(q.size) * (hi - lo)
    keep = (x > lo) & (x < hi)
    np.testing.assert_array_equal(f16.ulp(x[keep]), (hi - lo)[keep])
