"""Pins of the oracle's number formats against library conversions and a
brute-force nearest-value search over every representable value."""

import math
from fractions import Fraction

import numpy as np
import torch

import pytest


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    return vals, bits.astype(np.uint16)


def _brute_round(x: float, values: np.ndarray, bits: np.ndarray) -> int:
    """Nearest representable value by exhaustive search, ties to the even
    pattern; overflow beyond the largest finite + half a spacing goes to inf."""
    finite = np.isfinite(values)
    vals = values[finite]
    bts = bits[finite]
    fx = Fraction(x)
    d = np.abs(vals - x)
    best = np.min(d)
    cand = np.nonzero(d <= best * (1 + 1e-12) + 1e-300)[0]
    exact = [(abs(Fraction(float(vals[c])) - fx), int(bts[c])) for c in cand]
    mind = min(e[0] for e in exact)
    ties = [b for dist, b in exact if dist == mind]
    # prefer +0 over -0 and the even significand on a genuine tie
    ties = sorted(set(ties))
    if len(ties) > 1:
        nz = [b for b in ties if b & 0x7FFF]
        if not nz:
            return 0x8000 if x < 0 or (x == 0 and math.copysign(1, x) < 0) else 0
        ties = [b for b in ties if (b & 1) == 0] or ties
    return ties[0]


def test_bf16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ours = orc.half_bits_to_double(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_fp16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ours = orc.half_bits_to_double(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert np.array_equal(np.signbit(ours[m]), np.signbit(ref[m]))


def test_bf16_round_matches_torch_on_fp32_values(orc):
    # Values exactly representable in fp32: torch's fp32 -> bf16 conversion is
    # round-to-nearest-even, so the single rounding from double must agree.
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = words.view(np.float32)
    f = f[np.isfinite(f)]
    specials = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38, 3.4028235e38,
                         1e-45, -1e-45, 1.1754942e-38, 1.0039062, 1.0117188, 1.0078125,
                         1.00390625, 1.01171875], dtype=np.float32)
    f = np.concatenate([f, specials])
    ours = orc.double_to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_brute_force_ties_and_double_precision(orc):
    values, bits = _all_bf16_values()
    rng = np.random.default_rng(11)
    xs = []
    # exact midpoints between neighbouring bf16 values (ties -> even)
    for b in rng.integers(0, 0x7F7F, size=300):
        lo = values[b]
        hi = values[b + 1]
        xs += [(lo + hi) / 2, -(lo + hi) / 2]
    # values a hair off the midpoint (double-rounding traps through fp32)
    for b in rng.integers(1, 0x7F7F, size=300):
        lo = values[b]
        hi = values[b + 1]
        mid = (lo + hi) / 2
        xs += [np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    xs += [1e-41, 3e-40, -7e-39, 6e-45, 1e-46]  # subnormal range
    for x in xs:
        got = int(orc.double_to_bf16_bits(np.array([x]))[0])
        assert got == _brute_round(float(x), values, bits), x


def test_bf16_round_overflow_and_nan(orc):
    mx = float(np.float32(3.3895314e38))  # largest finite bf16
    spacing = 2.0 ** (127 - 7)
    below = orc.double_to_bf16_bits(np.array([np.nextafter(mx + spacing / 2, 0.0)]))[0]
    at = orc.double_to_bf16_bits(np.array([mx + spacing / 2]))[0]
    assert below == 0x7F7F
    assert at == 0x7F80  # tie rounds to the even pattern, which is +inf
    assert orc.double_to_bf16_bits(np.array([-1e300]))[0] == 0xFF80
    nan = orc.double_to_bf16_bits(np.array([np.nan]))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_fp16_round_matches_numpy(orc):
    # numpy converts float64 -> float16 with a single round-to-nearest-even.
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100_000) * 10.0 ** rng.integers(-9, 6, size=100_000),
        np.array([65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0**-24, 2.0**-25, 2.0**-25 * 1.0000001,
                  3 * 2.0**-26, 0.0, -0.0, 6.1035156e-05]),
    ])
    ours = orc.double_to_fp16_bits(x)
    with np.errstate(over="ignore"):  # values beyond the fp16 range round to +-inf on purpose
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
