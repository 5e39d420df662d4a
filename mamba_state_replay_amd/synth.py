"""Seeded synthetic inputs for the Mamba-2 decode workloads.

This module only draws random numbers and rounds them to the storage types the
layer consumes.  It holds none of the layer's arithmetic: both the HIP path and
the fp64 oracle receive exactly the arrays produced here.

Distributions follow the Nemotron-3-style Mamba-2 layer shape that the ReplaySSM
blog post uses as its running example (NVIDIA Developer blog "ReplaySSM ...",
section "State memory traffic": one layer's FP32 state is 4 MiB per sequence,
i.e. nheads=128 x headdim=64 x dstate=128 x 4 B):

* x, B, C ~ N(0, 1), stored as fp32 or rounded to bf16 (round to nearest even)
* dt = softplus(N(0, 1) - 2), fp32 (dt is handed over after the softplus)
* A = -exp(U(0, ln 16)) per head, fp32 (negative, so exp(dt*A) is a decay)
* D ~ N(0, 1) per head, fp32
* initial checkpoint ~ N(0, 0.1) fp32 (0.1 read as the standard deviation), or 0
* accepted draft counts ~ U{0..T}

Per decode step the draw order is x, B, C, dt; acceptance counts for a
speculative round are drawn after that round's draft inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 1000


@dataclass(frozen=True)
class LayerShape:
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    window: int = 16       # L, records per window before a flush
    max_drafts: int = 1    # T_max

    @property
    def cap(self) -> int:
        """Ring capacity of the input-record buffer (L + 2*T_max - 1)."""
        return self.window + 2 * self.max_drafts - 1


# The workloads: tiny correctness case, the headline Nemotron-3-style layer, and
# the variants of that layer used for verification and dual precision.
TINY = LayerShape(batch=1, nheads=4, headdim=16, dstate=16, ngroups=1, window=4)
NEMOTRON3 = LayerShape(batch=256, nheads=128, headdim=64, dstate=128, ngroups=8,
                       window=16)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tokens:
    """Per-token layer inputs for `steps` consecutive tokens.

    x  [steps][batch][nheads][headdim]
    B  [steps][batch][ngroups][dstate]
    C  [steps][batch][ngroups][dstate]
    dt [steps][batch][nheads] (fp32, post-softplus)

    `x`, `B`, `C` hold the values as fp32 (already rounded when the storage
    type is bf16); `x_bits` etc. hold the bf16 bit patterns in that case.
    """
    x: np.ndarray
    B: np.ndarray
    C: np.ndarray
    dt: np.ndarray
    in_dtype: str
    x_bits: np.ndarray | None = None
    B_bits: np.ndarray | None = None
    C_bits: np.ndarray | None = None

    @property
    def steps(self) -> int:
        return self.x.shape[0]

    def storage(self, name: str) -> np.ndarray:
        """The array in the layout and type the device consumes."""
        if self.in_dtype == "bf16":
            return getattr(self, name + "_bits")
        return getattr(self, name)

    def slice(self, t0: int, t1: int) -> "Tokens":
        def s(a):
            return None if a is None else a[t0:t1]
        return Tokens(self.x[t0:t1], self.B[t0:t1], self.C[t0:t1], self.dt[t0:t1],
                      self.in_dtype, s(self.x_bits), s(self.B_bits), s(self.C_bits))


def _store(a: np.ndarray, in_dtype: str):
    a = a.astype(np.float32)
    if in_dtype == "bf16":
        bits = bf16_bits(a)
        return bf16_to_f32(bits), bits
    if in_dtype == "f32":
        return a, None
    raise ValueError(f"unknown input dtype {in_dtype!r}")


def softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def draw_dt(g: np.random.Generator, size) -> np.ndarray:
    return softplus(g.standard_normal(size) - 2.0).astype(np.float32)


def layer_params(g: np.random.Generator, nheads: int):
    """A = -exp(U(0, ln 16)), D ~ N(0, 1), one of each per head (fp32)."""
    A = (-np.exp(g.uniform(0.0, np.log(16.0), nheads))).astype(np.float32)
    D = g.standard_normal(nheads).astype(np.float32)
    return A, D


def tokens(g: np.random.Generator, steps: int, shape: LayerShape,
           in_dtype: str = "bf16") -> Tokens:
    """Draw `steps` tokens; per step the order is x, B, C, dt."""
    b, nh, hd, ds, ng = shape.batch, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    xs, Bs, Cs, dts = [], [], [], []
    for _ in range(steps):
        xs.append(g.standard_normal((b, nh, hd), dtype=np.float32))
        Bs.append(g.standard_normal((b, ng, ds), dtype=np.float32))
        Cs.append(g.standard_normal((b, ng, ds), dtype=np.float32))
        dts.append(draw_dt(g, (b, nh)))
    x, xb = _store(np.stack(xs) if steps else np.zeros((0, b, nh, hd), np.float32), in_dtype)
    B, Bb = _store(np.stack(Bs) if steps else np.zeros((0, b, ng, ds), np.float32), in_dtype)
    C, Cb = _store(np.stack(Cs) if steps else np.zeros((0, b, ng, ds), np.float32), in_dtype)
    dt = np.stack(dts) if steps else np.zeros((0, b, nh), np.float32)
    return Tokens(x, B, C, dt, in_dtype, xb, Bb, Cb)


def checkpoint(g: np.random.Generator, shape: LayerShape, std: float = 0.1) -> np.ndarray:
    """Initial FP32 checkpoint [batch][nheads][headdim][dstate]."""
    size = (shape.batch, shape.nheads, shape.headdim, shape.dstate)
    if std == 0.0:
        return np.zeros(size, np.float32)
    return (g.standard_normal(size, dtype=np.float32) * np.float32(std)).astype(np.float32)


def acceptance(g: np.random.Generator, batch: int, T: int) -> np.ndarray:
    """Accepted draft count per sequence, U{0..T} (int32)."""
    return g.integers(0, T + 1, size=batch, dtype=np.int64).astype(np.int32)


def staggered_fill(batch: int, window: int) -> np.ndarray:
    """Committed records per sequence for staggered phases: 1 + (b mod L)."""
    return (1 + (np.arange(batch) % window)).astype(np.int32)


@dataclass
class Workload:
    """A whole seeded run: parameters, initial state and the token stream.

    `pre` holds the tokens already sitting in the buffer when the run starts
    (sequence b has its first `n0[b]` of them committed); `steps` holds the
    tokens fed to the decode calls.
    """
    shape: LayerShape
    A: np.ndarray
    D: np.ndarray
    h0: np.ndarray
    n0: np.ndarray
    pre: Tokens
    steps: Tokens
    extra: dict = field(default_factory=dict)


def decode_workload(shape: LayerShape, nsteps: int, seed: int, in_dtype: str = "bf16",
                    ckpt_std: float = 0.1, n0=None) -> Workload:
    """Parameters, checkpoint, pre-filled records and `nsteps` decode tokens.

    `n0` is an int (same fill for every sequence), an int array, or None for an
    empty buffer.
    """
    g = rng(seed)
    A, D = layer_params(g, shape.nheads)
    h0 = checkpoint(g, shape, ckpt_std)
    if n0 is None:
        n0 = np.zeros(shape.batch, np.int32)
    elif np.isscalar(n0):
        n0 = np.full(shape.batch, int(n0), np.int32)
    n0 = np.asarray(n0, np.int32)
    pre = tokens(g, int(n0.max()) if n0.size else 0, shape, in_dtype)
    steps = tokens(g, nsteps, shape, in_dtype)
    return Workload(shape, A, D, h0, n0, pre, steps)


def verify_workload(shape: LayerShape, rounds: int, T: int, seed: int,
                    in_dtype: str = "bf16", ckpt_std: float = 0.1, n0=None) -> Workload:
    """Speculative rounds: T draft tokens then the accepted counts, per round.

    Stored as `steps` with rounds*T tokens (round r's drafts are tokens
    r*T .. r*T+T-1) and `extra["accepted"]` [rounds][batch].
    """
    g = rng(seed)
    A, D = layer_params(g, shape.nheads)
    h0 = checkpoint(g, shape, ckpt_std)
    if n0 is None:
        n0 = g.integers(0, shape.window, size=shape.batch).astype(np.int32)
    elif np.isscalar(n0):
        n0 = np.full(shape.batch, int(n0), np.int32)
    n0 = np.asarray(n0, np.int32)
    pre = tokens(g, int(n0.max()) if n0.size else 0, shape, in_dtype)
    parts, acc = [], []
    for _ in range(rounds):
        parts.append(tokens(g, T, shape, in_dtype))
        acc.append(acceptance(g, shape.batch, T))
    steps = _concat(parts, shape, in_dtype)
    return Workload(shape, A, D, h0, n0, pre, steps,
                    extra={"accepted": np.stack(acc) if acc else np.zeros((0, shape.batch), np.int32),
                           "T": T})


def _concat(parts, shape, in_dtype) -> Tokens:
    if not parts:
        return tokens(rng(0), 0, shape, in_dtype)

    def cat(name):
        vals = [getattr(p, name) for p in parts]
        return None if vals[0] is None else np.concatenate(vals)
    return Tokens(cat("x"), cat("B"), cat("C"), cat("dt"), in_dtype,
                  cat("x_bits"), cat("B_bits"), cat("C_bits"))
