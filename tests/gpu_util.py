"""Helpers for the GPU parity tests (compare HIP results with the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = 1e-4  # max relative error of FP32-state outputs vs the fp64 oracle


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be attributed."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def rel_err_rows(got: np.ndarray, ref: np.ndarray, axis=-1) -> np.ndarray:
    """max_i |got - ref| / max_i |ref| along `axis` (one value per output row)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=axis)
    den = np.max(np.abs(ref), axis=axis)
    return num / np.maximum(den, 1e-30)


ROW_FLOOR = 1e-2  # a row's normaliser is at least this fraction of its head's output scale


def head_err(got, ref) -> np.ndarray:
    """Normalized error per (sequence, head): max |got - ref| over every token and
    headdim output of that head, divided by max |ref| over the same outputs (a
    diagnostic printed beside the per-row check below).

    Arrays are [...tokens...][batch][nheads][headdim]."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    axes = tuple(range(got.ndim - 3)) + (got.ndim - 1,)
    num = np.abs(got - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    return num / np.maximum(den, 1e-30)


def row_norm(ref) -> np.ndarray:
    """Normaliser of each (sequence, head, token) row: max_i |ref| over the row's
    headdim outputs, floored at ROW_FLOOR times the head's output scale (max |ref|
    over every token and output of that head).  A row can be near zero through
    cancellation of O(1)-O(10) terms, where its own maximum measures only the
    rounding of those terms; the floor keeps such a row to 1e-2 of the head's
    scale instead."""
    ref = np.abs(np.asarray(ref, np.float64))
    axes = tuple(range(ref.ndim - 3)) + (ref.ndim - 1,)
    scale = ref.max(axis=axes, keepdims=True)[..., 0]           # [1..][batch][nheads]
    return np.maximum(ref.max(axis=-1), ROW_FLOOR * scale)


def row_err(got, ref, allowance=None) -> np.ndarray:
    """Per-row error max_i (|got - ref| - allowance_i)^+ / row_norm(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    if allowance is not None:
        diff = np.maximum(diff - np.asarray(allowance, np.float64), 0.0)
    return diff.max(axis=-1) / np.maximum(row_norm(ref), 1e-30)


def assert_rows_close(got, ref, tol=TOL, what="outputs", allowance=None):
    """Every (sequence, head, token) row within tol of the oracle: max_i |got - ref|
    <= tol * row_norm(ref) (+ allowance_i where a stated bound adds one, e.g. the
    fp16 spacing of a half-precision checkpoint).  Arrays are
    [...tokens...][batch][nheads][headdim]."""
    got = np.asarray(got)
    assert got.shape == np.asarray(ref).shape, (got.shape, np.asarray(ref).shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = row_err(got, ref, allowance)
    worst = float(err.max()) if err.size else 0.0
    per_head = head_err(got, ref)
    raw = rel_err_rows(got, ref)
    print(f"[gpu] {what}: max error per row (floored) {worst:.2e}; per head {float(per_head.max()) if per_head.size else 0.0:.2e}, "
          f"worst unfloored row {float(raw.max()) if raw.size else 0.0:.2e}", flush=True)
    assert worst <= tol, (f"{what}: max normalized row error {worst:.3e} > {tol:.1e} at "
                          f"{np.unravel_index(err.argmax(), err.shape)}")
    return worst


def tile_err(got, ref):
    """Per-tile error of states [batch][nheads][hd][ds], normalized by the tile max."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=(-1, -2))
    den = np.abs(ref).max(axis=(-1, -2))
    return num / np.maximum(den, 1e-30)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda", 0)
