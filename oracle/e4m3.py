"""FP8 E4M3 decode and encode, written from the format's definition.

Test infrastructure (see the package docstring): not part of the product path.

Reading of the pages: they call the element type "e4m3" / "f8e4m3" (Linnet
"Backend plugins" page, DeepGemm.match in the plugin source; deepgemm-rust
README, "What's implemented" table) and convert with round-to-nearest and
saturation to the largest finite value ("cvt.rn.satfinite", deepgemm-rust
README, "Blackwell-native FP4/FP8" key techniques).  We take the OCP "FN"
variant of E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, a single NaN pattern per sign (exponent and mantissa all ones),
largest finite magnitude 448.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
# Half-way between 448 and the next step of the exponent-15 binade (480): the
# encoder saturates at and above this magnitude.
_SATURATE_FROM = 464.0


def _code_value(code: int) -> float:
    """The real value of one E4M3 byte, from its bit fields."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return float("nan")
    if exponent == 0:
        # subnormal: (m / 8) * 2^(1 - bias)
        return sign * (mantissa / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


def e4m3_table() -> np.ndarray:
    """float64[256]: the value of every byte (NaN for 0x7F and 0xFF)."""
    return np.array([_code_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()
# Non-negative finite values in code order 0x00..0x7E; they increase with the code.
_POSITIVE = _TABLE[:0x7F].copy()
assert np.all(np.diff(_POSITIVE) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of E4M3 bytes (uint8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3 bytes: nearest finite value, ties to the
    even code, magnitudes of 464 and above saturate to 448, the sign bit is
    copied (so -0 and negative underflow give 0x80).  NaN maps to 0x7F (it lies
    outside the path's contract)."""
    y = np.asarray(y, dtype=np.float32)
    mag = np.abs(y).astype(np.float64)  # exact
    nan = np.isnan(mag)
    mag = np.where(nan, 0.0, mag)
    # candidates: the table values just below and just above the magnitude
    hi = np.searchsorted(_POSITIVE, mag, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POSITIVE[lo]
    d_hi = _POSITIVE[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(mag >= _SATURATE_FROM, 0x7E, code)
    code = code.astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    return code
