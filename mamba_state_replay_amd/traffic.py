"""Algorithmic HBM bytes of the decode-path kernels (measurement accounting).

Counts what each call must move at minimum, per sequence:

  E    = nheads*headdim*dstate            state elements
  S    = 4E (FP32) or 2E (FP16)           checkpoint (or conventional state) bytes
  S_r  = bytes of the tile a non-flush call reads: S, 2E (bf16 copy),
         E + nheads*4 (e4m3 copy + per-tile scales), E/2 + E/32 (MXFP4
         codes + one E8M0 byte per 32 elements) or E + E/32 (MXFP8)
  S_c  = read-copy bytes a flush writes (0 without a copy)
  R    = nheads*headdim*e + ngroups*dstate*e + nheads*4   one record (x, B, dt)
  TOK  = R + ngroups*dstate*e                             one token's inputs (+ C)
  Y    = nheads*headdim*4                                 one token's outputs

  replay decode, non-flush, n records: S_r + n*R + TOK + R + Y
  replay decode, flush of n records:   S + n*R + TOK + S + S_c + R + Y
  replay verify of T drafts:           S_r + n*R + T*(TOK + R + Y)   (+ S + S_c, S_r -> S on a flush)
  conventional step:                   2*S + TOK + Y
  snapshot verify of T drafts:         (1 + T)*S + T*(TOK + Y)

e is the input element size (2 for bf16).  The 1 KiB of per-head A and D and
the 8-byte ring pointers are ignored.  The realized schedule (which calls
flush, and how many records each reads) is replayed here with the same
integer rule as the kernels: a call that starts with n >= L flushes first.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Sizes:
    S: int
    S_r: int
    S_c: int
    R: int
    TOK: int
    Y: int


def sizes(nheads, headdim, dstate, ngroups, in_bytes=2, read_copy=None, ckpt_bytes=4) -> Sizes:
    """Per-sequence sizes; ckpt_bytes = 4 for the FP32 checkpoint, 2 for FP16."""
    E = nheads * headdim * dstate                  # state elements per sequence
    S = E * ckpt_bytes
    if read_copy is None:
        S_r, S_c = S, 0
    elif read_copy == "bf16":
        S_r = S_c = 2 * E
    elif read_copy == "e4m3":
        S_r = S_c = E + nheads * 4
    elif read_copy == "mxfp4":
        S_r = S_c = E // 2 + E // 32
    elif read_copy == "mxfp8":
        S_r = S_c = E + E // 32
    else:
        raise ValueError(read_copy)
    R = nheads * headdim * in_bytes + ngroups * dstate * in_bytes + nheads * 4
    TOK = R + ngroups * dstate * in_bytes
    Y = nheads * headdim * 4
    return Sizes(S, S_r, S_c, R, TOK, Y)


def decode_schedule(n0: np.ndarray, L: int, steps: int):
    """Per step: (records read n [batch], flushed [batch]) under flush-at-start."""
    n = np.array(n0, np.int64).copy()
    out = []
    for _ in range(steps):
        fold = n >= L
        out.append((n.copy(), fold.copy()))
        n = np.where(fold, 0, n) + 1
    return out, n


def decode_step_bytes(sz: Sizes, n: np.ndarray, fold: np.ndarray) -> int:
    """Algorithmic bytes of one replay decode call over the batch."""
    nonfold = sz.S_r + n * sz.R + sz.TOK + sz.R + sz.Y
    folded = sz.S + n * sz.R + sz.TOK + sz.S + sz.S_c + sz.R + sz.Y
    return int(np.where(fold, folded, nonfold).sum())


def conventional_step_bytes(sz: Sizes, batch: int) -> int:
    return batch * (2 * sz.S + sz.TOK + sz.Y)


def verify_bytes(sz: Sizes, n: np.ndarray, fold: np.ndarray, T: int) -> int:
    base = n * sz.R + T * (sz.TOK + sz.R + sz.Y)
    return int(np.where(fold, base + 2 * sz.S + sz.S_c, base + sz.S_r).sum())


def snapshot_verify_bytes(sz: Sizes, batch: int, T: int) -> int:
    return batch * ((1 + T) * sz.S + T * (sz.TOK + sz.Y))


def gdn_sizes(nv, nk, dk, dv, in_bytes=2, ckpt_bytes=4) -> Sizes:
    """Per-sequence sizes of a Gated DeltaNet layer in the same accounting:
    S = nv*dv*dk*ckpt_bytes (4 FP32, 2 FP16); a record is the key (per key
    head, in the input type), the corrected value u (per value head, fp32) and
    g (fp32); a token's inputs are q, k (per key head), v (per value head), g
    and beta; outputs are fp32."""
    S = nv * dv * dk * ckpt_bytes
    R = nk * dk * in_bytes + nv * dv * 4 + nv * 4
    TOK = 2 * nk * dk * in_bytes + nv * dv * in_bytes + 2 * nv * 4
    Y = nv * dv * 4
    return Sizes(S, S, 0, R, TOK, Y)
