"""Pins of the oracle's E4M3FN decoding (format definition; library cross-check)."""

import math

import numpy as np
import pytest

from oracle import E4M3FN_TABLE, decode_e4m3fn


def test_named_values():
    # largest finite, smallest normal, smallest subnormal, +-1, zero, NaN
    assert E4M3FN_TABLE[0x7E] == 448.0
    assert E4M3FN_TABLE[0x08] == 2.0 ** -6
    assert E4M3FN_TABLE[0x01] == 2.0 ** -9
    assert E4M3FN_TABLE[0x38] == 1.0
    assert E4M3FN_TABLE[0xB8] == -1.0
    assert E4M3FN_TABLE[0x00] == 0.0 and E4M3FN_TABLE[0x80] == 0.0
    assert math.copysign(1.0, E4M3FN_TABLE[0x80]) == -1.0
    assert math.isnan(E4M3FN_TABLE[0x7F]) and math.isnan(E4M3FN_TABLE[0xFF])
    assert np.isnan(E4M3FN_TABLE).sum() == 2


def test_all_codes_match_library_conversion():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = E4M3FN_TABLE
    nan = np.isnan(lib)
    assert (nan == np.isnan(ours)).all()
    assert np.array_equal(lib[~nan], ours[~nan])


def test_monotone_and_symmetric():
    pos = E4M3FN_TABLE[:0x7F]
    assert (np.diff(pos) > 0).all()                     # codes 0..126 increase
    assert np.array_equal(E4M3FN_TABLE[0x80:0xFF], -E4M3FN_TABLE[:0x7F])


def test_integers_exact():
    # every integer in [-8, 8] is representable; the integer-grid workloads rely on it
    vals = set(E4M3FN_TABLE[~np.isnan(E4M3FN_TABLE)].tolist())
    for i in range(-8, 9):
        assert float(i) in vals


def test_nan_rejected():
    with pytest.raises(ValueError):
        decode_e4m3fn(np.array([0x38, 0x7F], np.uint8))
