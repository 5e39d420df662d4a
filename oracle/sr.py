"""FP16 recurrence checkpoint with stochastic rounding: the oracle side.

TEST INFRASTRUCTURE ONLY: the tests use this module; the library never does.

NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
Hybrid-Model Decoding", section "Benefit 3: Limit error accumulation with
separate precisions": a flush starts from the recurrence checkpoint, folds the
buffered records in and writes the result; an FP16 recurrence checkpoint is
enough when that write rounds stochastically.  The pages fix neither the
random source nor the rounding's resolution; the reading used here (and by the
library) is:

* random words: Philox4x32-10, the counter-based generator of Salmon, Moraes,
  Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011),
  written here from that definition;
* checkpoint element 4 v + e (row-major over the whole [batch][nheads]
  [headdim][dstate] array, v its 4-element vector) draws 16 bits from word e
  of Philox under the key (seed mod 2^32, seed div 2^32), one seed per call:
  within each aligned block of 32 vectors (128 elements), vectors v and
  v + 16 (v mod 32 < 16) share the counter (u mod 2^32, u div 2^32, 0, 0)
  with u = 16 (v div 32) + (v mod 16); the lower vector takes the low 16 bits
  of each word, the upper one the high 16 bits.  Each generator call thus
  serves 8 elements (the rounding below uses 13 bits of a draw);
* stochastic rounding of a value v to fp16 with random draw r: let a be the
  fp16 grid point at or below |v| and s the grid spacing there (2^(E - 10) for
  |v| in [2^E, 2^(E+1)), E >= -14; 2^-24 below 2^-14), d the distance
  (|v| - a) / s taken to 13 bits (rounded down); |v| goes to a + s iff
  d + (r mod 2^13) >= 2^13, else to a; the sign is kept, |v| >= 65504 gives
  65504, NaN stays NaN.  In the fp16 normal range d is exact, so the result's
  expectation over r is v itself.

The exact fold is the definition's stepping (oracle.conventional) in fp64
from the previous checkpoint's fp16 values; `sr_checkpoint` rounds it.
"""
from __future__ import annotations

import numpy as np

_MASK = 0xFFFFFFFF
_M0, _M1 = 0xD2511F53, 0xCD9E8D57          # round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85          # key increments (Weyl sequence)
F16_MAX = 65504.0


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 on arrays of 32-bit counter words (any integer dtype);
    returns the four output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(w).astype(np.uint64) & np.uint64(_MASK) for w in (c0, c1, c2, c3)]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    k0, k1 = int(k0) & _MASK, int(k1) & _MASK
    m0, m1, mask = np.uint64(_M0), np.uint64(_M1), np.uint64(_MASK)
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = m0 * c0                                       # < 2^64: both factors < 2^32
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return c0, c1, c2, c3


def counter(v):
    """Generator counter of 4-element vector v (vectors v and v + 16 of an
    aligned block of 32 share one)."""
    v = np.asarray(v, np.uint64)
    return (v >> np.uint64(5)) * np.uint64(16) + (v & np.uint64(15))


def words(index, seed: int) -> np.ndarray:
    """Random 16-bit draw of each checkpoint element (flat row-major index array)."""
    idx = np.asarray(index, np.uint64)
    v = idx >> np.uint64(2)
    u = counter(v)
    out = philox4x32_10(u & np.uint64(_MASK), u >> np.uint64(32), 0, 0, seed & _MASK, (seed >> 32) & _MASK)
    w = np.stack(out)                                      # [4][...]
    e = (idx & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(w, e[None], axis=0)[0]
    shift = ((v >> np.uint64(4)) & np.uint64(1)) * np.uint64(16)
    return ((word >> shift) & np.uint64(0xFFFF)).astype(np.uint32)


def f16_grid(a):
    """(grid point at or below, spacing) of the fp16 grid at a >= 0 (finite, float64)."""
    a = np.asarray(a, np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))              # a = m 2^ex, m in [0.5, 1)
    spacing = np.where(a >= 2.0 ** -14, np.ldexp(1.0, ex - 11), 2.0 ** -24)
    below = np.floor(a / spacing) * spacing                # exact: spacing is a power of two
    return below, spacing


def f16_sr(v, r) -> np.ndarray:
    """Stochastic rounding of v (float32 values) to fp16 with random draws r
    (integers, the low 13 bits used); float64 results, all on the fp16 grid
    (NaN for NaN)."""
    v = np.asarray(v, np.float32).astype(np.float64)
    r13 = (np.asarray(r, np.uint64) & np.uint64(0x1FFF)).astype(np.int64)
    a = np.abs(v)
    fin = np.where(np.isfinite(a), np.minimum(a, F16_MAX), F16_MAX)
    below, s = f16_grid(fin)
    d = np.floor((fin - below) / s * 8192.0).astype(np.int64)
    mag = below + np.where(d + r13 >= 8192, s, 0.0)
    mag = np.minimum(mag, F16_MAX)
    out = np.copysign(mag, v)
    return np.where(np.isnan(v), np.nan, out)


def sr_checkpoint(h_exact, seed: int) -> np.ndarray:
    """The FP16 checkpoint a flush writes for the exact state h_exact
    ([batch][nheads][headdim][dstate]), as float64 values on the fp16 grid.
    The decision is taken on h_exact rounded to fp32 (the precision the
    kernel's registers hold)."""
    h = np.asarray(h_exact, np.float64)
    idx = np.arange(h.size, dtype=np.uint64).reshape(h.shape)
    return f16_sr(h.astype(np.float32), words(idx, seed))
