"""OCP 8-bit floating point, E4M3 variant ("E4M3FN"), for the quantised latent cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): never imported by the library.

The pages motivate quantising the latent as a whole: on page keybo.xyz,
"MLA 之后，KV cache 确实得重新理解一遍", section "所以 cache 逻辑到底哪里要重写",
quantising c_kv spreads its error over every head, and K and V cannot be
quantised apart because they come from the same latent.  The pages give no
format; the format below is the OCP "8-bit Floating Point Specification (OFP8)"
E4M3 encoding, written from that definition:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent 0: subnormal, value m * 2^-9;
* otherwise (1 + m/8) * 2^(e-7);
* exponent 15 with mantissa 7 is NaN; there are no infinities; the largest
  finite magnitude is 448.

Quantisation of one cache row (reading chosen where the pages are silent):
one float32 scale per token over all its values, s = amax / 448 in float32
(s = 1 when the row is all zero); each value is x / s in float32, then encoded
to the nearest E4M3 value, ties to the even code, saturating at +-448.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(code) -> np.ndarray:
    """Value of each E4M3 code (float64; NaN for the NaN codes)."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.power(2.0, e - 7.0)
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def _magnitude_table():
    """All finite non-negative codes 0x00..0x7E with their values (ascending)."""
    codes = np.arange(0x7F, dtype=np.int64)
    return codes, decode(codes)


def encode(x) -> np.ndarray:
    """Nearest E4M3 code to each float32 value; ties go to the even code;
    magnitudes above 448 saturate to 448; the sign bit copies x's sign."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    codes, vals = _magnitude_table()
    mag = np.minimum(np.abs(x), MAX_FINITE)
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    pick_hi |= hi == lo
    mcode = np.where(pick_hi, codes[hi], codes[lo])
    sign = np.signbit(x).astype(np.int64) << 7
    return (mcode | sign).astype(np.uint8)


def quantize_rows(rows) -> tuple[np.ndarray, np.ndarray]:
    """Quantise each row (float32 values) with its own float32 scale.

    Returns (codes uint8 [T, D], scales float32 [T]).
    """
    r = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(r), axis=1)
    s = np.where(amax > 0, amax / np.float32(MAX_FINITE), np.float32(1.0)).astype(np.float32)
    y = (r / s[:, None]).astype(np.float32)
    return encode(y), s


def dequantize_rows(codes, scales) -> np.ndarray:
    """x = s * decode(code), exactly, in float64."""
    return decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]
