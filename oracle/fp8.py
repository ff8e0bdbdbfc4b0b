"""OCP FP8 E4M3 (the "e4m3fn" variant) and the KV quantiser, from their definitions.

Quantising the KV cache to FP8 is the pages' capacity lever for decode (Blog
#54, section 4: KV quantisation to FP8 or INT4; Part 8, quantisation section:
FP8 E4M3 halves the KV cache). The pages fix neither the encoding variant nor
the scale granularity; the readings taken here:
  * encoding: OCP E4M3 -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity;
    largest finite 448;
  * rounding: to nearest, ties to even, on the fp32 value;
  * scales: one fp32 scale per (token, KV head): the smallest power of two
    that is >= amax / 448 over that token's head vector (the quotient taken in
    fp32; 1 for an all-zero vector), code = round(x / scale) (exact division
    by a power of two, then the rounding above). The dequantised value is
    decode(code) * scale. A power-of-two scale (like the shared exponents of
    the OCP microscaling formats) changes no code's relative precision, and a
    weight times it stays a bf16 number, so attention applies it exactly.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
# finite non-negative codes sorted by value (0x00..0x7E), for encoding
_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)
_POS_VALS = _TABLE[_POS_CODES]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> codes, round to nearest, ties to the even code.

    Magnitudes up to 464 round to the largest finite value 448 (464 is the tie
    between 448 and the next step, and 448's code is even); larger ones have
    no finite code. The quantiser's x / scale can exceed 448 by one fp32 ulp.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    if np.any(a > 464.0) or np.any(np.isnan(a)):
        raise ValueError("e4m3_encode: value outside the finite range")
    hi = np.searchsorted(_POS_VALS, a, side="left")       # first representable >= a
    hi = np.minimum(hi, _POS_VALS.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    exact = _POS_VALS[hi] == a
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    # the sign is kept, also for values that round to zero (-0 is code 0x80)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def pow2_ceil(s: np.ndarray) -> np.ndarray:
    """The smallest power of two >= s, elementwise, for fp32 s > 0."""
    s = np.asarray(s, dtype=np.float32)
    frac, e = np.frexp(s.astype(np.float64))  # s = frac * 2^e, frac in [0.5, 1)
    return np.where(frac == 0.5, s.astype(np.float64), np.ldexp(1.0, e)).astype(np.float32)


def quantize_rows(x: np.ndarray):
    """Quantise the last axis of fp32 x: returns (codes uint8 like x, scales fp32 x.shape[:-1])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    q = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax > 0, pow2_ceil(np.where(amax > 0, q, np.float32(1.0))), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values: decode(code) * scale (scales broadcast over the last axis)."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]
