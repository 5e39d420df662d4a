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


# ---------------------------------------------------------------------------
# MXFP4 (OCP Microscaling formats, version 1.0): blocks of 32 elements share
# one E8M0 scale X = 2^(e - 127) (e = 255 is NaN); the elements are FP4 E2M1
# (1 sign, 2 exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3,
# 4, 6; no infinity, no NaN).  The scale of a block is X = 2^(floor(log2 amax)
# - 2), 2 being the largest exponent of E2M1, so amax / X lies in [4, 8); the
# elements are v / X rounded to the nearest E2M1 value (ties to even code),
# saturating at +-6.  Here: X is clamped to 2^-126 .. 2^127 (e = 1 .. 254, so
# the scale is always a normal fp32 number; a block of zeros or of values below
# 2^-124 gets e = 1), and a block holding a NaN gets e = 255.
# ---------------------------------------------------------------------------
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.int64)
    v = E2M1[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(a) -> np.ndarray:
    """Nearest E2M1 code of a (float64, already divided by the scale), ties to
    the even code, saturating at +-6."""
    a = np.asarray(a, np.float64)
    m = np.minimum(np.abs(a), 6.0)
    hi = np.clip(np.searchsorted(E2M1, m), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    dlo, dhi = m - E2M1[lo], E2M1[hi] - m
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(a), 8, 0)).astype(np.uint8)


def e8m0_value(e) -> np.ndarray:
    e = np.asarray(e, np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def mxfp4_encode(x) -> tuple[np.ndarray, np.ndarray]:
    """fp32 array [..., 32 k] -> (E8M0 scales [..., k] uint8, E2M1 codes
    [..., 32 k] uint8, one code per byte)."""
    x = np.asarray(x, np.float32)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1).astype(np.float32)          # NaN if the block holds one
    biased = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    e = np.clip(biased - 2, 1, 254)
    e = np.where(np.isnan(amax), 255, e)
    X = e8m0_value(e)
    codes = e2m1_encode(blk.astype(np.float64) / np.where(np.isnan(X), 1.0, X)[..., None])
    return e.astype(np.uint8), codes.reshape(x.shape)


def mxfp4_decode(scales, codes) -> np.ndarray:
    c = np.asarray(codes)
    v = e2m1_decode(c).reshape(c.shape[:-1] + (c.shape[-1] // 32, 32))
    return (v * e8m0_value(scales)[..., None]).reshape(c.shape)


def mxfp8_scale(amax) -> np.ndarray:
    """E8M0 byte of an MXFP8 block scale, from its definition: the smallest
    power of two X = 2^(e - 127) with amax / X <= 448 (e clamped to 1..254);
    255 for a NaN; an infinite amax is taken as the largest finite fp32."""
    a = np.asarray(amax, np.float64)
    fin = np.where(np.isnan(a), 0.0, np.minimum(a, float(np.finfo(np.float32).max)))
    k = np.ceil(np.log2(np.where(fin > 0, fin, 1.0) / 448.0)).astype(np.int64)
    # guard the floating-point log: X = 2^k must hold amax, 2^(k-1) must not (448 * 2^k is exact)
    k = np.where(fin > 448.0 * np.exp2(k.astype(np.float64)), k + 1, k)
    k = np.where(fin <= 448.0 * np.exp2(k.astype(np.float64) - 1.0), k - 1, k)
    e = np.clip(k + 127, 1, 254)
    e = np.where(fin == 0, 1, e)
    return np.where(np.isnan(a), 255, e).astype(np.int64)


def mxfp8_encode(x) -> tuple[np.ndarray, np.ndarray]:
    """fp32 array [..., 32 k] -> (E8M0 scales [..., k] uint8, e4m3fn codes
    [..., 32 k] uint8): each block's codes encode v / X (exact division by a
    power of two), nearest even; a NaN block keeps X = 1 for its codes."""
    x = np.asarray(x, np.float32)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1).astype(np.float32)
    e = mxfp8_scale(amax)
    X = e8m0_value(e)
    codes = encode_e4m3fn(blk.astype(np.float64) / np.where(np.isnan(X), 1.0, X)[..., None])
    return e.astype(np.uint8), codes.reshape(x.shape)


def mxfp8_decode(scales, codes) -> np.ndarray:
    c = np.asarray(codes)
    v = decode_e4m3fn(c).reshape(c.shape[:-1] + (c.shape[-1] // 32, 32))
    return (v * e8m0_value(scales)[..., None]).reshape(c.shape)


def e2m1_encode_fast(x) -> np.ndarray:
    """Same as e2m1_encode for fp32 input (no NaN), by counting the midpoints
    passed: a tie at a midpoint goes to the even code (the thresholds at
    0.75, 1.75 and 3.5 are inclusive, those at 0.25, 1.25, 2.5 and 5 are not)."""
    x = np.asarray(x, np.float32)
    a = np.abs(x)
    code = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
            + (a > 5.0)).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 3)
