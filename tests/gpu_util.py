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


def head_err(got, ref) -> np.ndarray:
    """Normalized error per (sequence, head): max |got - ref| over every token and
    headdim output of that head, divided by max |ref| over the same outputs.

    Arrays are [...tokens...][batch][nheads][headdim].  A single output row can
    be near zero through cancellation of O(1) terms, where a row-relative error
    measures only fp32 rounding of those terms; the head's output scale is the
    meaningful yardstick."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    axes = tuple(range(got.ndim - 3)) + (got.ndim - 1,)
    num = np.abs(got - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    return num / np.maximum(den, 1e-30)


def assert_rows_close(got, ref, tol=TOL, what="outputs"):
    """All outputs within tol of the oracle, normalized per (sequence, head)."""
    got = np.asarray(got)
    assert got.shape == np.asarray(ref).shape, (got.shape, np.asarray(ref).shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = head_err(got, ref)
    worst = float(err.max()) if err.size else 0.0
    rows = rel_err_rows(got, ref)
    print(f"[gpu] {what}: max error per head {worst:.2e}, worst single row {float(rows.max()):.2e}",
          flush=True)
    assert worst <= tol, f"{what}: max normalized error {worst:.3e} > {tol:.1e} at (seq, head) {np.unravel_index(err.argmax(), err.shape)}"
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
