"""The host format definitions agree with torch's float8_e4m3fn and bfloat16."""
import numpy as np
import torch

from tests import formats


def test_e4m3fn_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    val, nan = formats.e4m3fn_table()
    assert np.array_equal(np.isnan(ref), nan)
    assert np.array_equal(ref[~nan], val[~nan])
    assert val[~nan].max() == 448.0 and val[0x01] == 2.0 ** -9 and val[0x08] == 2.0 ** -6


def test_e4m3fn_encoding_matches_torch_in_range():
    g = np.random.default_rng(0)
    val, nan = formats.e4m3fn_table()
    finite = np.sort(np.unique(val[~nan]))
    mids = (finite[1:] + finite[:-1]) / 2          # every tie between neighbours
    x = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                        g.uniform(-448, 448, 20000), np.exp(g.uniform(-14, 6, 20000)) * g.choice([-1, 1], 20000)])
    x = x.astype(np.float32)
    ours = formats.encode_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.all(formats.same_code(ours, ref))


def test_e4m3fn_saturates_and_nan():
    codes = formats.encode_e4m3fn(np.array([448.0, 460.0, 1e9, -1e9, np.inf, np.nan]))
    assert list(codes[:5]) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E] and codes[5] == 0x7F


def test_decode_roundtrip():
    val, nan = formats.e4m3fn_table()
    codes = np.arange(256)[~nan]
    assert np.all(formats.same_code(formats.encode_e4m3fn(formats.decode_e4m3fn(codes)), codes))


def _bf16_probe_bits(g):
    """Random fp32 patterns, every exponent with the rounding-boundary low
    halves (ties with even and odd kept bit, one below, one above), zeros,
    infinities, the largest finite values and NaNs."""
    rnd = g.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    hi = (np.arange(2 ** 16, dtype=np.uint32) << 16)
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    edges = (hi[:, None] | lows[None, :]).ravel()
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000,
                        0x7F7F7FFF, 0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x00000001, 0x00008000], np.uint32)
    return np.concatenate([rnd, edges, special])


def test_bf16_encoder_matches_torch():
    """The host bf16 encoder against torch's fp32 -> bf16 conversion (round to
    nearest even) on every exponent's rounding boundaries and random patterns."""
    g = np.random.default_rng(5)
    bits = _bf16_probe_bits(g)
    ours = formats.encode_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan_ours, nan_ref = formats.bf16_is_nan(ours), formats.bf16_is_nan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])


def test_fast_e4m3_encoder_matches_table_encoder():
    """The arithmetic e4m3fn encoder used for exhaustive checks equals the
    table encoder written from the format definition: on every fp32 within
    2 ulp of each e4m3 value and of each midpoint, and on random values."""
    g = np.random.default_rng(6)
    val, nan = formats.e4m3fn_table()
    fin = np.unique(val[~nan])
    pts = np.concatenate([fin, (fin[1:] + fin[:-1]) / 2]).astype(np.float32)
    near = pts.view(np.int32)[:, None] + np.arange(-2, 3, dtype=np.int32)[None, :]
    near = near.ravel().view(np.float32)
    rnd = np.concatenate([g.uniform(-500, 500, 500_000), np.exp(g.uniform(-25, 6.2, 500_000)) *
                          g.choice([-1.0, 1.0], 500_000)]).astype(np.float32)
    x = np.concatenate([near, rnd, np.array([np.nan, -np.nan, 0.0, -0.0, 448.0, 464.0, 1e30], np.float32)])
    assert np.array_equal(formats.encode_e4m3fn_fast(x), formats.encode_e4m3fn(x))


def test_e2m1_codes_and_rounding():
    """Every E2M1 code decodes to its value and encodes back to itself; the
    midpoints between neighbours go to the even code; magnitudes above 6
    saturate; the sign is kept on zero."""
    codes = np.arange(16)
    vals = formats.e2m1_decode(codes)
    assert np.array_equal(np.abs(vals[:8]), [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    back = formats.e2m1_encode(vals)
    assert np.array_equal(back, codes.astype(np.uint8))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert np.array_equal(formats.e2m1_encode(mids), [0, 2, 2, 4, 4, 6, 6])
    assert np.array_equal(formats.e2m1_encode(-mids), np.array([0, 2, 2, 4, 4, 6, 6]) | 8)
    assert np.array_equal(formats.e2m1_encode([6.5, 8.0, 1e30, -7.0]), [7, 7, 7, 15])
    near = np.nextafter(mids, 0.0), np.nextafter(mids, 10.0)
    assert np.array_equal(formats.e2m1_encode(near[0]), [0, 1, 2, 3, 4, 5, 6])
    assert np.array_equal(formats.e2m1_encode(near[1]), [1, 2, 3, 4, 5, 6, 7])


def test_mxfp4_block_scale_and_error():
    """The block scale puts amax / X in [4, 8); every element's decode error is
    at most |v| / 4 + X / 4 (the bound the read-copy tests use); a block of
    zeros gets the smallest normal scale 2^-126 and zero codes; a NaN makes
    the scale NaN."""
    g = np.random.default_rng(11)
    x = (np.exp(g.uniform(-20, 20, (500, 1))) * g.standard_normal((500, 128))).astype(np.float32)
    e, c = formats.mxfp4_encode(x)
    X = formats.e8m0_value(e)
    amax = np.abs(x.reshape(500, 4, 32)).max(axis=-1)
    big = amax >= 2.0 ** -124                 # below it the scale is clamped at 2^-126
    assert np.all((amax / X >= 4) & (amax / X < 8) | ~big)
    dec = formats.mxfp4_decode(e, c)
    err = np.abs(dec - x.astype(np.float64))
    Xe = np.repeat(X, 32, axis=-1)
    assert np.all(err <= np.abs(x) / 4 + Xe / 4)
    z = np.zeros((1, 32), np.float32)
    ez, cz = formats.mxfp4_encode(z)
    assert ez[0, 0] == 1 and np.all(cz == 0)
    n = np.ones((1, 32), np.float32)
    n[0, 7] = np.nan
    en, _ = formats.mxfp4_encode(n)
    assert en[0, 0] == 255 and np.all(np.isnan(formats.mxfp4_decode(en, _)))
    # a worked block: amax 5 -> floor(log2 5) = 2 -> X = 2^0; codes are the E2M1 encodings of v
    w = np.array([[5.0, -0.3, 0.25, 0.75, 2.6, 3.4, 1.0, -6.0] + [0.0] * 24], np.float32)
    ew, cw = formats.mxfp4_encode(w)
    assert ew[0, 0] == 127
    assert list(cw[0, :8]) == [6, 9, 0, 2, 5, 5, 2, 15]


def test_mxfp8_block_scale_and_error():
    """The MXFP8 block scale is the smallest power of two X with amax / X <=
    448, so amax / X lies in (224, 448] and nothing saturates; every element's
    decode error is at most |v| / 16 + X / 1024 (half the e4m3 spacing,
    relative in the normal range, absolute below it); worked scales at the
    edges of the rule; zeros, NaN and infinity."""
    g = np.random.default_rng(13)
    x = (np.exp(g.uniform(-20, 20, (500, 1))) * g.standard_normal((500, 128))).astype(np.float32)
    e, c = formats.mxfp8_encode(x)
    X = formats.e8m0_value(e)
    amax = np.abs(x.reshape(500, 4, 32)).max(axis=-1).astype(np.float64)
    big = amax >= 2.0 ** -117                 # below it the scale is clamped at 2^-126
    r = amax / X
    assert np.all((r > 224) & (r <= 448) | ~big)
    dec = formats.mxfp8_decode(e, c)
    err = np.abs(dec - x.astype(np.float64))
    Xe = np.repeat(X, 32, axis=-1)
    assert np.all(err <= np.abs(x) / 16 + Xe / 1024)
    # worked scales: 448 fits X = 1; the next fp32 above needs X = 2; 1.0 and 1.75 fit 2^-8
    # (256 and 448), the fp32 just above 1.75 needs 2^-7; 0 -> the smallest normal scale
    f32 = np.float32
    cases = {448.0: 127, float(np.nextafter(f32(448), f32(1e9))): 128, 1.0: 119, 1.75: 119,
             float(np.nextafter(f32(1.75), f32(2))): 120, 0.0: 1, float("inf"): 247, 2.0 ** -130: 1}
    for a, want in cases.items():
        assert formats.mxfp8_scale(np.float32(a)) == want, (a, want)
    n = np.ones((1, 32), np.float32)
    n[0, 3] = np.nan
    en, cn = formats.mxfp8_encode(n)
    assert en[0, 0] == 255 and np.all(np.isnan(formats.mxfp8_decode(en, cn)))
    # a worked block: amax 3.0 -> X = 2^-7 (3 * 128 = 384 <= 448, 3 * 256 > 448); codes encode v * 128
    w = np.array([[3.0, -1.0, 0.5, 2.0 ** -9] + [0.0] * 28], np.float32)
    ew, cw = formats.mxfp8_encode(w)
    assert ew[0, 0] == 120
    assert np.array_equal(formats.decode_e4m3fn(cw[0, :4]), [384.0, -128.0, 64.0, 0.25])


def test_fast_e2m1_encoder_matches_definition():
    """The midpoint-counting E2M1 encoder used for exhaustive checks equals the
    nearest-value encoder on every fp32 within 2 ulp of each value, midpoint
    and the saturation point, and on random values."""
    g = np.random.default_rng(12)
    pts = np.concatenate([formats.E2M1, (formats.E2M1[1:] + formats.E2M1[:-1]) / 2, [7.0, 8.0]]).astype(np.float32)
    near = (pts.view(np.int32)[:, None] + np.arange(-2, 3, dtype=np.int32)[None, :]).ravel().view(np.float32)
    x = np.concatenate([near, -near, g.uniform(-9, 9, 1_000_000).astype(np.float32)])
    x = x[np.isfinite(x)]                     # steps below +0 land on NaN patterns
    assert np.array_equal(formats.e2m1_encode_fast(x), formats.e2m1_encode(x))
