"""Pins of the oracle's E4M3 cache codes (oracle/fp8.py) against what the
format fixes: the closed-form value of each code, PyTorch's float8_e4m3fn
conversion (a library routine) inside the range where it does not saturate
to NaN, exact round trips, ties to even and saturation.  A planted mistake
(ties away from zero) fails the library pin."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def test_code_values_closed_form():
    v = fp8.e4m3_values()
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x07] == 7 / 8 * 2.0 ** -6
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:127]) > 0)                 # increasing over 0 .. 448
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])  # sign symmetry


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.e4m3_decode(np.arange(256))
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), ~fin)
    assert np.array_equal(ours[fin], ref[fin])


def test_encode_matches_torch_float8_in_range():
    """PyTorch's cast turns magnitudes of 464 and more (half-way to the next
    binade) into NaN; below that both round to nearest, ties to even."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 60, 20000), rng.uniform(-463.9, 463.9, 5000),
                        rng.normal(0, 2 ** -7, 5000)]).astype(np.float32)
    x = x[np.abs(x) < 464]
    # exact midpoints between neighbouring codes exercise the ties
    v = fp8.e4m3_values()[:127]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_round_trip_ties_and_saturation():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(finite)), np.array(finite, dtype=np.uint8))
    # ties go to the even mantissa: 1 + 1/16 lies between 1 (0x38) and 1.125 (0x39)
    assert fp8.e4m3_encode(1.0625) == 0x38 and fp8.e4m3_encode(1.1875) == 0x3A
    # saturation: finite values past 448 store +-448, never NaN
    assert fp8.e4m3_encode(480.0) == 0x7E and fp8.e4m3_encode(-1e30) == 0xFE
    assert fp8.e4m3_encode(float("nan")) == 0x7F


def test_quantize_divides_in_fp32():
    x = np.array([3.0, -7.5, 0.1], dtype=np.float32)
    s = np.float32(0.37)
    assert np.array_equal(fp8.quantize(x, s), fp8.e4m3_encode(x / s))
    assert np.allclose(fp8.dequantize(fp8.quantize(x, s), s), x, rtol=2 ** -4)


def test_planted_tie_mistake_fails_the_library_pin(monkeypatch):
    v = fp8.e4m3_values()[:127]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)

    def away_from_zero(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.minimum(np.abs(x), 448.0)
        i = np.searchsorted(v, a)
        return np.where(np.isclose(a, v[np.maximum(i - 1, 0)]), np.maximum(i - 1, 0), np.minimum(i, 126)).astype(np.uint8)

    monkeypatch.setattr(fp8, "e4m3_encode", away_from_zero)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(fp8.e4m3_encode(mids), ref)
