"""Pins for the oracle's OCP E4M3 codec: values fixed by the OFP8 format
definition (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals,
no infinities, one NaN pattern per sign, largest finite 448), exhaustive
round trips, tie-to-even midpoints, and an independent implementation
(torch's float8_e4m3fn) where one exists."""
import numpy as np
import pytest

from oracle import e4m3 as E


def test_decode_fixed_points():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0,
             0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in table.items():
        assert E.decode(code) == val, hex(code)
    assert np.signbit(E.decode(0x80)) and E.decode(0x80) == 0.0
    nan_codes = [c for c in range(256) if np.isnan(E.decode(c))]
    assert nan_codes == [0x7F, 0xFF]
    finite = E.decode(np.arange(256))
    finite = finite[~np.isnan(finite)]
    assert np.abs(finite).max() == 448.0 and len(finite) == 254


def test_decode_matches_torch_float8():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = E.decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(ours))


def test_encode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(E.encode(E.decode(codes).astype(np.float32)), codes.astype(np.uint8))


def test_encode_ties_to_even_and_saturation():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 1.5 * 2.0 ** -9: 0x02,
             -1.0625: 0xB8, 1000.0: 0x7E, -1e30: 0xFE, 449.0: 0x7E, 464.0: 0x7E,
             1.06: 0x38, 1.07: 0x39}
    for x, code in cases.items():
        assert int(E.encode(np.float32(x))) == code, x


def test_encode_matches_torch_float8_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 9, 200000)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(E.encode(x), ref)


def test_quantize_rows_scale_and_error_bound():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((300, 576)).astype(np.float32)
    rows[0] = 0.0
    codes, s = E.quantize_rows(rows)
    assert s[0] == 1.0 and np.all(codes[0] == 0)
    amax = np.abs(rows[1:]).max(axis=1)
    assert np.array_equal(s[1:], (amax / np.float32(448)).astype(np.float32))
    # the largest element of each row lands on +-448
    arg = np.abs(rows[1:]).argmax(axis=1)
    assert np.all(np.abs(E.decode(codes[1:][np.arange(299), arg])) == 448.0)
    # round-to-nearest error: half a step of the E4M3 grid at that magnitude
    deq = E.dequantize_rows(codes, s)
    y = np.abs(rows / s[:, None]).astype(np.float64)
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    assert np.all(np.abs(deq - rows) <= 0.5 * step * s[:, None] * (1 + 1e-6))
