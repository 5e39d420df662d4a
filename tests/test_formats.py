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
