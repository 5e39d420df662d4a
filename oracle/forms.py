"""Independent fp64 forms of the ReplaySSM computation, for self-checks.

TEST INFRASTRUCTURE ONLY (see oracle/oracle.c).  These forms let the tests
confirm, in fp64 and on the CPU, the readings of the formulas that extraction
stripped from the pages, against the step-by-step definition in oracle.c:

* replay form: the state over a window of records is the checkpoint decayed
  by the cumulative decay plus a decayed sum of the buffered rank-1 inputs
  (NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
  Hybrid-Model Decoding", section "How ReplaySSM represents the state");
* fold: a flush turns checkpoint + records into a new checkpoint (same
  section: the flush folds the buffered inputs into the checkpoint);
* output-only form: outputs of T queries from the checkpoint read once, a
  causally masked matrix of decays W applied to the scores C K^T, and the
  cached values (section "Benefit 2: Simplify rollback and speed up
  verification");
* ReplayModel: a checkpoint + record list driven by decode / verify / commit /
  flush with the flush taken at the start of a call once L records are
  committed (the pages only place the flush at the point where the buffer holds
  L records, and let it fold committed records alone).

Every function works on one (sequence, head) tile:
  Hs [headdim][dstate]; records x [n][headdim], B [n][dstate], dt [n];
  queries x [T][headdim], B [T][dstate], C [T][dstate], dt [T]; A, D scalars.
"""
from __future__ import annotations

import numpy as np


def _f64(*arrs):
    return [np.asarray(a, np.float64) for a in arrs]


def replay_outputs(Hs, rx, rB, rdt, A, D, qx, qB, qC, qdt):
    """Outputs of queries 0..T-1; query q sits at position n+q of the window.

    y_q = exp(sum_{k<=m} a_k) (Hs C_q)
          + sum_{k<=m} dt_k exp(sum_{k<i<=m} a_i) (B_k . C_q) x_k + D x_q,
    with m = n+q, a_k = dt_k A, and the sums of a taken as segment sums.
    """
    Hs, rx, rB, rdt, qx, qB, qC, qdt = _f64(Hs, rx, rB, rdt, qx, qB, qC, qdt)
    X = np.concatenate([rx.reshape(-1, Hs.shape[0]), qx])
    K = np.concatenate([rB.reshape(-1, Hs.shape[1]), qB])
    dts = np.concatenate([rdt.reshape(-1), qdt])
    a = dts * float(A)
    n = rdt.size
    ys = []
    for q in range(qdt.size):
        m = n + q
        y = np.exp(a[: m + 1].sum()) * (Hs @ qC[q])
        for k in range(m + 1):
            seg = a[k + 1: m + 1].sum()
            y = y + dts[k] * np.exp(seg) * float(K[k] @ qC[q]) * X[k]
        ys.append(y + float(D) * qx[q])
    return np.array(ys).reshape(qdt.size, Hs.shape[0])


def replay_fold(Hs, rx, rB, rdt, A):
    """New checkpoint after folding records 0..n-1 into Hs."""
    Hs, rx, rB, rdt = _f64(Hs, rx, rB, rdt)
    a = rdt.reshape(-1) * float(A)
    n = a.size
    H = np.exp(a.sum()) * Hs
    for k in range(n):
        H = H + rdt.reshape(-1)[k] * np.exp(a[k + 1:].sum()) * np.outer(rx[k], rB[k])
    return H


def output_only(Hs, rx, rB, rdt, A, D, qx, qB, qC, qdt):
    """Matrix form Y = diag(d) (C_Q Hs^T) + (W * (C_Q K^T)) X + D X_Q.

    d_q = exp(Lam_{n+q}); W[q,k] = dt_k exp(Lam_{n+q} - Lam_k) for k <= n+q,
    else 0; Lam is the prefix sum of a over the window (records, then queries).
    Uses prefix sums (unlike replay_outputs) so the two are independent.
    """
    Hs, rx, rB, rdt, qx, qB, qC, qdt = _f64(Hs, rx, rB, rdt, qx, qB, qC, qdt)
    X = np.concatenate([rx.reshape(-1, Hs.shape[0]), qx])
    K = np.concatenate([rB.reshape(-1, Hs.shape[1]), qB])
    dts = np.concatenate([rdt.reshape(-1), qdt])
    n, T = rdt.size, qdt.size
    lam = np.cumsum(dts * float(A))
    rows = n + np.arange(T)
    d = np.exp(lam[rows])
    mask = np.arange(n + T)[None, :] <= rows[:, None]
    expo = np.where(mask, lam[rows][:, None] - lam[None, :], 0.0)
    W = np.where(mask, dts[None, :] * np.exp(expo), 0.0)
    S = qC @ K.T
    return d[:, None] * (qC @ Hs.T) + (W * S) @ X + float(D) * qx


class ReplayModel:
    """Checkpoint + committed records, for one (sequence, head), in fp64.

    Policy: a call that starts with at least L committed records first folds
    all of them (fold at start); verify appends T drafts past the pointer and
    leaves the pointer alone; commit(a) keeps the first a drafts; decode is
    verify(1) followed by commit(1).
    """

    def __init__(self, Hs, A, D, L):
        self.Hs = np.array(Hs, np.float64)
        self.A, self.D, self.L = float(A), float(D), int(L)
        hd, ds = self.Hs.shape
        self.rx = np.zeros((0, hd))
        self.rB = np.zeros((0, ds))
        self.rdt = np.zeros(0)
        self.drafts = None
        self.folds = 0

    @property
    def n(self):
        return self.rdt.size

    def flush(self):
        if self.n:
            self.Hs = replay_fold(self.Hs, self.rx, self.rB, self.rdt, self.A)
            self.rx, self.rB, self.rdt = self.rx[:0], self.rB[:0], self.rdt[:0]
            self.folds += 1

    def state(self):
        """The canonical state: checkpoint with every committed record folded."""
        return replay_fold(self.Hs, self.rx, self.rB, self.rdt, self.A)

    def verify(self, qx, qB, qC, qdt):
        if self.n >= self.L:
            self.flush()
        qx, qB, qC, qdt = _f64(qx, qB, qC, qdt)
        y = replay_outputs(self.Hs, self.rx, self.rB, self.rdt, self.A, self.D,
                           qx, qB, qC, qdt)
        self.drafts = (qx, qB, qdt)
        return y

    def commit(self, a):
        qx, qB, qdt = self.drafts
        assert 0 <= a <= qdt.size
        self.rx = np.concatenate([self.rx, qx[:a]])
        self.rB = np.concatenate([self.rB, qB[:a]])
        self.rdt = np.concatenate([self.rdt, qdt[:a]])
        self.drafts = None

    def decode(self, x, B, C, dt):
        y = self.verify(np.asarray(x)[None], np.asarray(B)[None], np.asarray(C)[None],
                        np.asarray([dt]))
        self.commit(1)
        return y[0]
