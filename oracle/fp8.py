"""FP8 E4M3FN decoding, written from the format's definition (oracle; test infrastructure only).

The ECHO page (§2, DSA indexer) states that the indexer's q and k are FP8 but
not which FP8.  Reading: the OCP 8-bit E4M3 "FN" encoding (finite-only, one
NaN mantissa pattern, no infinities), which is the native FP8 of the target
hardware.  Fields of a byte b: sign = bit 7, exponent e = bits 6..3 (bias 7),
mantissa m = bits 2..0.

* e == 0            -> (-1)^sign * 2^(1-7) * (m / 8)          (subnormal)
* e == 15 and m == 7 -> NaN                                  (the only NaN)
* otherwise          -> (-1)^sign * 2^(e-7) * (1 + m / 8)     (max 448)

Pinned by: all 256 codes against torch's float8_e4m3fn conversion (a library
routine), and the named values 448, 2^-6, 2^-9, +-1, NaN.
"""

import numpy as np


def _decode_one(b: int) -> float:
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** (1 - 7)) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


# value of every byte, float64
E4M3FN_TABLE = np.array([_decode_one(b) for b in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E4M3FN bytes (uint8) to float64.

    Raises ValueError if a NaN code is present: NaN is not a valid indexer
    input and would make every score it touches undefined.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    out = E4M3FN_TABLE[codes]
    if np.isnan(out).any():
        raise ValueError("E4M3FN NaN code in input")
    return out
