"""Seeded synthetic inputs for the Gated DeltaNet (GDN) decode workloads.

Random draws and their rounding to the storage types only; none of the
layer's arithmetic.  Both the HIP path and the fp64 oracle receive exactly
the arrays produced here.

The ReplaySSM page evaluates GDN layers (section "How we evaluated
ReplaySSM") but prints no GDN shape; the layer used here has 32 value heads
over 16 key heads with key and value head dimension 128 (FP32 state 2 MiB per
sequence, 64 KiB per head).  Per token, in this draw order:

* q, k ~ N(0, 1) per key head, each scaled to unit L2 norm over dk (the gated
  delta rule normalises its keys and queries), q then multiplied by
  1/sqrt(dk); rounded to bf16 (nearest even) or kept fp32
* v ~ N(0, 1) per value head, bf16 or fp32
* g = dt * A with dt = softplus(N(0, 1) - 2) and A = -exp(U(0, ln 16)) per
  value head (the same decay law as the Mamba-2 workloads), fp32
* beta = sigmoid(N(0, 1)), fp32
Initial checkpoint ~ N(0, 0.1) fp32 (0.1 the standard deviation) or 0;
accepted draft counts ~ U{0..T}.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .synth import _store, draw_dt, rng

SEED_BASE = 2000


@dataclass(frozen=True)
class GdnShape:
    batch: int
    nv: int            # value heads
    nk: int            # key heads (nv % nk == 0)
    dk: int
    dv: int
    window: int = 16   # L
    max_drafts: int = 1

    @property
    def cap(self) -> int:
        return self.window + 2 * self.max_drafts - 1


GDN_TINY = GdnShape(batch=2, nv=4, nk=2, dk=16, dv=32, window=4)
GDN_LAYER = GdnShape(batch=512, nv=32, nk=16, dk=128, dv=128, window=16)


@dataclass
class GdnTokens:
    """q, k [steps][batch][nk][dk]; v [steps][batch][nv][dv]; g, beta
    [steps][batch][nv].  Values as fp32 (already rounded for bf16); *_bits
    hold the bf16 patterns when in_dtype is bf16."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    in_dtype: str
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None

    @property
    def steps(self) -> int:
        return self.q.shape[0]

    def storage(self, name: str) -> np.ndarray:
        if self.in_dtype == "bf16" and name in ("q", "k", "v"):
            return getattr(self, name + "_bits")
        return getattr(self, name)


def _unit(a: np.ndarray) -> np.ndarray:
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def gdn_tokens(g: np.random.Generator, steps: int, shape: GdnShape, A: np.ndarray,
               in_dtype: str = "bf16") -> GdnTokens:
    b, nv, nk, dk, dv = shape.batch, shape.nv, shape.nk, shape.dk, shape.dv
    qs, ks, vs, gs, bs = [], [], [], [], []
    for _ in range(steps):
        qs.append(_unit(g.standard_normal((b, nk, dk))) / np.sqrt(dk))
        ks.append(_unit(g.standard_normal((b, nk, dk))))
        vs.append(g.standard_normal((b, nv, dv)))
        gs.append((draw_dt(g, (b, nv)) * A[None, :]).astype(np.float32))
        bs.append((1.0 / (1.0 + np.exp(-g.standard_normal((b, nv))))).astype(np.float32))

    def stack(xs, shp):
        return np.stack(xs).astype(np.float32) if steps else np.zeros((0,) + shp, np.float32)

    q, qb = _store(stack(qs, (b, nk, dk)), in_dtype)
    k, kb = _store(stack(ks, (b, nk, dk)), in_dtype)
    v, vb = _store(stack(vs, (b, nv, dv)), in_dtype)
    return GdnTokens(q, k, v, stack(gs, (b, nv)), stack(bs, (b, nv)), in_dtype, qb, kb, vb)


@dataclass
class GdnWorkload:
    shape: GdnShape
    A: np.ndarray
    S0: np.ndarray
    steps: GdnTokens
    extra: dict = field(default_factory=dict)


def gdn_workload(shape: GdnShape, nsteps: int, seed: int, in_dtype: str = "bf16",
                 ckpt_std: float = 0.1, T: int | None = None) -> GdnWorkload:
    """A per head, the initial checkpoint, then `nsteps` tokens (or, with T,
    `nsteps` rounds of T draft tokens each followed by its acceptance draw,
    stored token-major as steps = nsteps * T and extra["accepted"]
    [rounds][batch])."""
    g = rng(seed)
    A = (-np.exp(g.uniform(0.0, np.log(16.0), shape.nv))).astype(np.float32)
    size = (shape.batch, shape.nv, shape.dv, shape.dk)
    S0 = (np.zeros(size, np.float32) if ckpt_std == 0.0
          else (g.standard_normal(size, dtype=np.float32) * np.float32(ckpt_std)).astype(np.float32))
    if T is None:
        return GdnWorkload(shape, A, S0, gdn_tokens(g, nsteps, shape, A, in_dtype))
    rounds, acc = [], []
    for _ in range(nsteps):
        rounds.append(gdn_tokens(g, T, shape, A, in_dtype))
        acc.append(g.integers(0, T + 1, size=shape.batch).astype(np.int32))
    cat = {name: np.concatenate([getattr(r, name) for r in rounds])
           for name in ("q", "k", "v", "g", "beta")}
    bits = {name: (np.concatenate([getattr(r, name + "_bits") for r in rounds]) if in_dtype == "bf16" else None)
            for name in ("q", "k", "v")}
    toks = GdnTokens(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], in_dtype,
                     bits["q"], bits["k"], bits["v"])
    return GdnWorkload(shape, A, S0, toks, {"accepted": np.stack(acc), "T": T})
