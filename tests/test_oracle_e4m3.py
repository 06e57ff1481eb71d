"""Pins for the oracle's E4M3 decode table and encoder.

Anchors (none of them is the oracle's own code):
* torch's CPU float8_e4m3fn cast, a library implementation of the same OCP
  format (the AReno FP8 decode pull request checked its E4M3 decode the same
  way: a CPU decode against torch.float8_e4m3fn);
* closed forms of the format;
* exact rational rounding (tests/exact.py).
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.exact import e4m3_code, f32_fraction

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_256_codes_match_torch():
    ours = oracle.e4m3_decode(ALL)
    ref = torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_closed_forms():
    t = oracle.e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0**-9 and t[0x07] == 7 * 2.0**-9
    assert t[0x08] == 2.0**-6
    assert t[0x38] == 1.0 and t[0x39] == 1.125
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    pos = t[:0x80]
    assert np.sum(np.isfinite(pos) & (pos > 0)) == 126  # 0x01..0x7E
    assert np.all(np.diff(pos[:0x7F]) > 0)
    # every finite value times 2^9 is an integer (used by the exact-product pin)
    fin = t[np.isfinite(t)]
    assert np.all(fin * 512 == np.round(fin * 512))


def test_encode_round_trip_every_code():
    t = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = t[codes].astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


@pytest.mark.parametrize(
    "value,code",
    [
        (1.0625, 0x38),  # tie between 1.0 (0x38, even) and 1.125 (0x39)
        (1.1875, 0x3A),  # tie between 1.125 (0x39) and 1.25 (0x3A, even)
        (464.0, 0x7E),  # tie between 448 and the (non-finite) 480 step: saturates
        (465.0, 0x7E),
        (1e30, 0x7E),
        (-1e30, 0xFE),
        (449.0, 0x7E),
        (2.0**-10, 0x00),  # tie between 0 and 2^-9
        (1.5 * 2.0**-10, 0x01),
        (3 * 2.0**-10, 0x02),  # tie between 1*2^-9 and 2*2^-9 -> even (2)
        (-1e-9, 0x80),
        (-0.0, 0x80),
        (0.0, 0x00),
        (1e-40, 0x00),  # float32 subnormal
    ],
)
def test_encode_special_points(value, code):
    assert int(oracle.e4m3_encode(np.array([value], dtype=np.float32))[0]) == code


def _structured_f32(limit=464.0):
    """All float32 with |v| <= limit whose low 16 bits are in a set that puts
    values on, just above and just below every E4M3 rounding boundary."""
    hi = np.arange(0, 0x43E9, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    v = bits.view(np.float32)
    v = v[np.abs(v) <= limit]
    return np.concatenate([v, -v])


def test_encode_matches_torch_structured():
    v = _structured_f32()
    assert np.array_equal(oracle.e4m3_encode(v), torch_encode(v))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 0x43E80001, size=4_000_000, dtype=np.uint32)
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.e4m3_encode(v), torch_encode(v))


def test_encode_saturates_beyond_464():
    rng = np.random.default_rng(5)
    bits = rng.integers(0x43E80001, 0x7F800000, size=100_000, dtype=np.uint32)
    v = bits.view(np.float32)
    assert np.all(oracle.e4m3_encode(v) == 0x7E)
    assert np.all(oracle.e4m3_encode(-v) == 0xFE)


def test_encode_matches_exact_rational_rounding():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x44800000, size=3000, dtype=np.uint32)  # |v| up to 1024
    v = bits.view(np.float32)
    ours = oracle.e4m3_encode(v)
    for x, c in zip(v, ours):
        assert e4m3_code(f32_fraction(x), bool(np.signbit(x))) == int(c), float(x)


@pytest.mark.slow
def test_encode_matches_torch_exhaustive():
    """Every float32 bit pattern with |v| <= 464 (about 2.3e9 values, both
    signs), in chunks."""
    step = 1 << 24
    for start in range(0, 0x43E80001, step):
        bits = np.arange(start, min(start + step, 0x43E80001), dtype=np.uint32)
        v = bits.view(np.float32)
        assert np.array_equal(oracle.e4m3_encode(v), torch_encode(v)), hex(start)
        assert np.array_equal(oracle.e4m3_encode(-v), torch_encode(-v)), hex(start)
