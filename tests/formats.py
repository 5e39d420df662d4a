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
