"""Python side of the fp64 CPU oracle (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the library never does.

`conventional` is the definition: the Mamba-2 decode recurrence stepped one
token at a time in fp64 (NVIDIA Developer blog "ReplaySSM: Rethinking State
Storage for Faster Hybrid-Model Decoding", section "Why SSM layers can become a
decoding bottleneck").  The scenario helpers below only compose calls of it:

* decode: step the committed buffer records from the checkpoint, then every
  decode token (section "How ReplaySSM represents the state": the replayed
  outputs equal the stepped ones except for rounding);
* verify: the outputs of T drafts are those of stepping them one by one from
  the committed state, and committing `a` of them equals having stepped only
  those `a` (section "Benefit 2: Simplify rollback and speed up verification").
"""
from __future__ import annotations

import ctypes
import os
import time
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
LIBRARY = HERE / "liboracle.so"

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


class Oracle:
    """One loaded build of oracle.c."""

    def __init__(self, path: Path | str = LIBRARY):
        path = Path(path)
        if not path.exists():
            raise FileNotFoundError(
                f"{path} is missing; build it with `python -m oracle._build` "
                "or __graft_entry__.build()")
        self.path = path
        self.lib = ctypes.CDLL(str(path))
        f = self.lib.orc_conventional
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int] * 6 + [_ip] + [_dp] * 8 + [ctypes.c_int]
        self.lib.orc_num_threads.restype = ctypes.c_int
        self.lib.orc_num_threads.argtypes = []

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    def conventional(self, h0, x, B, C, dt, A, D, nsteps=None, outputs=True, threads=0):
        """Step the recurrence over `steps` tokens (fp64).

        h0 [batch][nheads][headdim][dstate]; x [steps][batch][nheads][headdim];
        B, C [steps][batch][ngroups][dstate]; dt [steps][batch][nheads];
        A, D [nheads]; nsteps [batch] or None.
        Returns (H [batch][nheads][headdim][dstate], y [steps][batch][nheads][headdim]
        or None).  Outputs of tokens past nsteps[b] are left as NaN.
        """
        H = np.array(h0, dtype=np.float64, order="C", copy=True)
        batch, nheads, headdim, dstate = H.shape
        x = np.ascontiguousarray(x, np.float64)
        B = np.ascontiguousarray(B, np.float64)
        C = np.ascontiguousarray(C, np.float64)
        dt = np.ascontiguousarray(dt, np.float64)
        A = np.ascontiguousarray(A, np.float64)
        D = np.ascontiguousarray(D, np.float64)
        steps = x.shape[0]
        ngroups = B.shape[2] if B.ndim == 4 else 1
        assert x.shape == (steps, batch, nheads, headdim), x.shape
        assert B.shape == (steps, batch, ngroups, dstate), B.shape
        assert C.shape == B.shape and dt.shape == (steps, batch, nheads)
        assert A.shape == (nheads,) and D.shape == (nheads,)
        y = np.full((steps, batch, nheads, headdim), np.nan) if outputs else None
        ns = None
        if nsteps is not None:
            ns = np.ascontiguousarray(nsteps, np.int32)
            assert ns.shape == (batch,)
        rc = self.lib.orc_conventional(
            batch, nheads, headdim, dstate, ngroups, steps,
            ns.ctypes.data_as(_ip) if ns is not None else None,
            H.ctypes.data_as(_dp), x.ctypes.data_as(_dp), B.ctypes.data_as(_dp),
            C.ctypes.data_as(_dp), dt.ctypes.data_as(_dp), A.ctypes.data_as(_dp),
            D.ctypes.data_as(_dp), y.ctypes.data_as(_dp) if y is not None else None,
            int(threads))
        if rc != 0:
            raise ValueError(f"orc_conventional rejected its arguments (rc={rc})")
        return H, y


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def conventional(*args, **kw):
    return default().conventional(*args, **kw)


# ---------------------------------------------------------------------------
# Scenarios built only from the definition above.
# ---------------------------------------------------------------------------

def _tok(tokens, t0, t1, seqs):
    sl = slice(None) if seqs is None else seqs
    return (tokens.x[t0:t1][:, sl], tokens.B[t0:t1][:, sl], tokens.C[t0:t1][:, sl],
            tokens.dt[t0:t1][:, sl])


def committed_state(work, seqs=None, orc: Oracle | None = None, threads=0):
    """State after the records already committed when the run starts."""
    orc = orc or default()
    sl = slice(None) if seqs is None else seqs
    h0 = work.h0[sl]
    n0 = work.n0[sl]
    x, B, C, dt = _tok(work.pre, 0, work.pre.steps, seqs)
    H, _ = orc.conventional(h0, x, B, C, dt, work.A, work.D, nsteps=n0,
                            outputs=False, threads=threads)
    return H


def decode(work, nsteps=None, seqs=None, orc: Oracle | None = None, threads=0):
    """Outputs of the first `nsteps` decode tokens and the state after them.

    Returns (y [nsteps][batch'][nheads][headdim], H [batch'][...]) in fp64 for
    the selected sequences `seqs` (an index array, or None for all).
    """
    orc = orc or default()
    nsteps = work.steps.steps if nsteps is None else nsteps
    H = committed_state(work, seqs, orc, threads)
    x, B, C, dt = _tok(work.steps, 0, nsteps, seqs)
    H, y = orc.conventional(H, x, B, C, dt, work.A, work.D, threads=threads)
    return y, H


def verify_rounds(work, rounds=None, seqs=None, orc: Oracle | None = None, threads=0):
    """Speculative rounds: outputs of every draft, then commit the accepted ones.

    Returns (y [rounds][T][batch'][nheads][headdim], H after the last commit).
    """
    orc = orc or default()
    T = work.extra["T"]
    acc = work.extra["accepted"]
    rounds = acc.shape[0] if rounds is None else rounds
    sl = slice(None) if seqs is None else seqs
    H = committed_state(work, seqs, orc, threads)
    ys = []
    for r in range(rounds):
        x, B, C, dt = _tok(work.steps, r * T, r * T + T, seqs)
        _, y = orc.conventional(H, x, B, C, dt, work.A, work.D, threads=threads)
        ys.append(y)
        H, _ = orc.conventional(H, x, B, C, dt, work.A, work.D,
                                nsteps=acc[r][sl], outputs=False, threads=threads)
    return np.stack(ys) if ys else np.zeros((0, T) + H.shape[:3]), H


def time_decode(work, seqs, nsteps, threads=0, orc: Oracle | None = None):
    """Wall time of `nsteps` decode tokens for the sequences `seqs` (seconds)."""
    orc = orc or default()
    H = np.array(work.h0[seqs], np.float64)
    x, B, C, dt = _tok(work.steps, 0, nsteps, seqs)
    t0 = time.perf_counter()
    orc.conventional(H, x, B, C, dt, work.A, work.D, threads=threads)
    return time.perf_counter() - t0


def available_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1
