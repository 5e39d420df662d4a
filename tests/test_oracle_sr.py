"""Pins of the stochastic-rounding oracle (oracle/sr.py), CPU only.

* Philox4x32-10 against the known-answer vectors published with the
  generator (Random123 distribution, kat_vectors: philox4x32_10);
* every finite fp16 value is left unchanged whatever the random word;
* by enumeration of all 2^13 random residues: the number that round away
  equals the 13-bit distance, so the expectation is v exactly in the fp16
  normal range (the point of stochastic rounding), and within 2^-13 of a
  spacing below it;
* the two candidates are numpy's fp16 neighbours of v (an independent grid);
* sign symmetry, saturation at 65504, NaN, and the element -> random draw map.
"""
import numpy as np
import pytest

from oracle import sr


@pytest.mark.parametrize("ctr,key,want", [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox_known_answers(ctr, key, want):
    got = sr.philox4x32_10(*[np.array([c]) for c in ctr], *key)
    assert tuple(int(w[0]) for w in got) == want


def test_fp16_values_are_fixed_points():
    bits = np.arange(1 << 16, dtype=np.uint16)
    v = bits.view(np.float16)
    v = v[np.isfinite(v)].astype(np.float32)
    g = np.random.default_rng(31)
    for r in (0, 1, 0x1FFF, 0xFFFFFFFF, *g.integers(0, 2 ** 32, 4)):
        out = sr.f16_sr(v, np.full(v.shape, r, np.uint64))
        assert np.array_equal(out, v.astype(np.float64))
        assert np.array_equal(np.signbit(out), np.signbit(v))


def _enumerate(v):
    """Results of f16_sr(v) for every residue 0..8191 of the random word: [len(v)][8192]."""
    v = np.asarray(v, np.float32)
    r = np.arange(8192, dtype=np.uint64)
    return sr.f16_sr(np.repeat(v[:, None], 8192, axis=1), np.broadcast_to(r, (v.size, 8192)))


def test_expectation_is_exact_in_the_normal_range():
    g = np.random.default_rng(32)
    v = (np.exp(g.uniform(np.log(2.0 ** -14), np.log(60000.0), 300)) * g.choice([-1, 1], 300)).astype(np.float32)
    out = _enumerate(v)
    assert np.array_equal(out.mean(axis=1), v.astype(np.float64))     # sum of 8192 grid values: exact


def test_expectation_below_the_normal_range():
    g = np.random.default_rng(33)
    v = (g.uniform(0, 2.0 ** -14, 300) * g.choice([-1, 1], 300)).astype(np.float32)
    out = _enumerate(v)
    err = np.abs(out.mean(axis=1) - v.astype(np.float64))
    assert np.all(err < 2.0 ** -24 * 2.0 ** -13)                       # the distance is taken to 13 bits


def test_candidates_are_the_fp16_neighbours():
    g = np.random.default_rng(34)
    v = np.concatenate([np.exp(g.uniform(-20, 11, 2000)), g.uniform(0, 2.0 ** -14, 200)]).astype(np.float32)
    v = v * g.choice([-1, 1], v.size).astype(np.float32)
    out = sr.f16_sr(v, g.integers(0, 2 ** 32, v.size).astype(np.uint64))
    n16 = v.astype(np.float16)                                        # nearest fp16 (numpy)
    lo = np.where(n16.astype(np.float64) > v, np.nextafter(n16, np.float16(-np.inf)), n16).astype(np.float64)
    hi = np.where(n16.astype(np.float64) < v, np.nextafter(n16, np.float16(np.inf)), n16).astype(np.float64)
    assert np.all((out == lo) | (out == hi))
    # and the count of draws that go up matches the distance (one value, all residues)
    one = np.float32(1.0 + 3 * 2.0 ** -13)                            # 3/8 of an fp16 spacing above 1
    ups = (_enumerate([one])[0] > 1.0).sum()
    assert ups == 3 * 2 ** 10


def test_sign_saturation_nan():
    g = np.random.default_rng(35)
    v = np.exp(g.uniform(-30, 11, 500)).astype(np.float32)
    r = g.integers(0, 2 ** 32, 500).astype(np.uint64)
    assert np.array_equal(sr.f16_sr(-v, r), -sr.f16_sr(v, r))
    big = np.array([65504, 65519, 65520, 70000, 1e30, np.inf, -np.inf], np.float32)
    out = sr.f16_sr(big, np.full(big.size, 0x1FFF, np.uint64))
    assert np.array_equal(out, np.copysign(65504.0, big.astype(np.float64)))
    assert np.isnan(sr.f16_sr(np.array([np.nan], np.float32), np.array([5], np.uint64)))[0]
    zero = sr.f16_sr(np.array([-0.0, -1e-30], np.float32), np.array([0, 0], np.uint64))
    assert np.all(zero == 0) and np.all(np.signbit(zero))


def test_element_words():
    """Element 4 v + e draws from word e of the generator: vectors v and v + 16
    of an aligned block of 32 share the counter 16 (v div 32) + (v mod 16), the
    lower vector taking the word's low 16 bits, the upper its high 16 bits."""
    seed = 0x0123456789ABCDEF
    vs = [0, 1, 15, 16, 17, 31, 32, 47, 48, 63, 1000, (1 << 32) + 7, (1 << 36) + 21]
    idx = np.array([4 * v + e for v in vs for e in range(4)], np.uint64)
    got = sr.words(idx, seed)
    for i, w in zip(idx.tolist(), got.tolist()):
        v, e = i // 4, i % 4
        block, pos = divmod(v, 32)
        u = block * 16 + pos % 16
        ref = sr.philox4x32_10(np.array([u & 0xFFFFFFFF]), np.array([u >> 32]), np.array([0]), np.array([0]),
                               seed & 0xFFFFFFFF, seed >> 32)
        word = int(ref[e][0])
        assert w == ((word >> 16) if pos >= 16 else word) & 0xFFFF
    # every counter serves exactly the 8 elements of one vector pair, and the two
    # halves of every word are used once each
    idx = np.arange(4 * 32 * 3, dtype=np.uint64)
    u = sr.counter(idx >> np.uint64(2))
    assert np.array_equal(np.bincount(u.astype(np.int64)), np.full(48, 8))


