"""Host encoders of the read-copy formats, written from their definitions.

bf16: the top 16 bits of an fp32 after round to nearest, ties to even.
e4m3fn (OCP 8-bit float E4M3, "fn" variant): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
S.1111.111 is NaN and there are no infinities, so the largest finite value is
1.75 * 2^8 = 448.  Encoding rounds to the nearest finite value, ties to the
even code, saturating at +-448.
"""
from __future__ import annotations

import numpy as np


def e4m3fn_table():
    """(value of every code 0..255 as float64, NaN mask)."""
    codes = np.arange(256)
    sign = codes >> 7
    exp = (codes >> 3) & 0xF
    man = codes & 0x7
    mag = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (exp - 7.0))
    val = np.where(sign == 1, -mag, mag)
    nan = (codes & 0x7F) == 0x7F
    return val, nan


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest e4m3fn code, ties to even, saturating at +-448; NaN -> 0x7F."""
    x = np.asarray(x, np.float64)
    val, nan = e4m3fn_table()
    pos = val[:0x7F]                       # codes 0..126: 0 .. 448, increasing
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(pos, a), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo = a - pos[lo]
    dhi = pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def decode_e4m3fn(codes) -> np.ndarray:
    val, nan = e4m3fn_table()
    out = val[np.asarray(codes, np.int64)]
    return np.where(nan[np.asarray(codes, np.int64)], np.nan, out)


def same_code(a, b) -> np.ndarray:
    """Codes equal, with +0 (0x00) and -0 (0x80) treated as one value."""
    a = np.asarray(a, np.int64)
    b = np.asarray(b, np.int64)
    return (a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))


def encode_bf16_bits(bits) -> np.ndarray:
    """bf16 bit patterns of fp32 bit patterns (uint32 array): round to nearest,
    ties to even, on the 16 dropped bits; values past the largest finite bf16
    round to infinity; a NaN stays a NaN (quieted, sign and top payload kept)."""
    b = np.asarray(bits, np.uint32)
    r = b + np.uint32(0x7FFF)
    r += (b >> np.uint32(16)) & np.uint32(1)       # wraps only for NaN patterns, replaced below
    r >>= np.uint32(16)
    nan = ((b & np.uint32(0x7F800000)) == np.uint32(0x7F800000)) & ((b & np.uint32(0x7FFFFF)) != 0)
    r[nan] = (b[nan] >> np.uint32(16)) | np.uint32(0x40)
    return r.astype(np.uint16)


def bf16_is_nan(h) -> np.ndarray:
    h = np.asarray(h, np.uint16).astype(np.uint32)
    return (((h >> 7) & 0xFF) == 0xFF) & ((h & 0x7F) != 0)


def encode_e4m3fn_fast(x) -> np.ndarray:
    """Same result as encode_e4m3fn for fp32 input, computed on the bits (for
    large arrays): in the normal range (|x| >= 2^-6) the 23 mantissa bits are
    rounded to 3 (nearest, ties to even), carrying into the exponent; below it
    the code is the subnormal count m = |x| 2^9 rounded to nearest even (m = 8
    is the smallest normal code), i.e. the 24-bit significand shifted right by
    14 - e; codes saturate at 0x7E (448); NaN gives 0x7F."""
    x = np.asarray(x, np.float32)
    b = x.view(np.uint32)
    mag = b & np.uint32(0x7FFFFFFF)
    e = (mag >> np.uint32(23)).astype(np.int32) - 127
    m = mag & np.uint32(0x7FFFFF)
    m3 = (m + np.uint32(0x7FFFF) + ((m >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)   # 0..8
    code = ((e + 7) << 3) + m3.astype(np.int32)                       # m3 = 8 carries into the exponent
    # subnormal range: significand (with the implicit bit) shifted right by 14 - e, to nearest even
    sh = np.clip(14 - e, 1, 25).astype(np.uint32)
    sig = (m | np.uint32(0x800000)) * (e > -127)                     # fp32 subnormals: below 2^-10, code 0
    q = sig >> sh
    rem = sig - (q << sh)
    half = np.uint32(1) << (sh - np.uint32(1))
    q = q + ((rem > half) | ((rem == half) & ((q & np.uint32(1)) == 1)))
    code = np.where(e < -6, q.astype(np.int32), code)
    code = np.minimum(code, 0x7E)
    code |= ((b >> np.uint32(31)) << np.uint32(7)).astype(np.int32)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)
