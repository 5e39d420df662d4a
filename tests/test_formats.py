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
