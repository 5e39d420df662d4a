"""Pins of the oracle's scenario functions (committed_state, decode, verify_rounds).

Every Mamba-2 GPU parity test takes its expected values from these three
functions, so each is checked here against two computations that share no code
with them:

* the brute-force closed form of the recurrence (tests/oracle_pins.brute_force:
  products of per-step decay factors, no recurrence), applied to the token
  stream each sequence actually commits;
* oracle.forms.ReplayModel, the checkpoint + record-buffer model driven by
  decode / verify / commit with its own flushes (NVIDIA Developer blog
  "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding",
  section "Benefit 2: Simplify rollback and speed up verification": a commit
  only moves the buffer pointer over the accepted prefix, so committing `a`
  drafts equals having decoded just those `a`).

The workloads are tiny but have every feature the GPU tests rely on:
per-sequence committed records at the start (n0), windows short enough that
the model folds several times, acceptance drawn from U{0..T}, and a selection
of sequences (`seqs`).  Each pin takes the oracle module (or a copy of it with a
planted mistake, see test_oracle_scenarios.py) and the loaded oracle library,
and raises AssertionError on a mismatch.
"""
from __future__ import annotations

import numpy as np

from mamba_state_replay_amd import synth
from oracle import forms
from tests.oracle_pins import brute_force

TOL = 1e-10
SHAPE = synth.LayerShape(batch=4, nheads=4, headdim=6, dstate=8, ngroups=2, window=3, max_drafts=3)


def _close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    err = float(np.max(np.abs(got - ref))) / scale if ref.size else 0.0
    assert err <= TOL, f"{what}: normalized error {err:.3e} > {TOL:.0e}"


def _stream(tok, t0, t1, b):
    """Tokens t0..t1-1 of sequence b as a one-sequence stream [steps][1][...]."""
    return (tok.x[t0:t1, b:b + 1], tok.B[t0:t1, b:b + 1], tok.C[t0:t1, b:b + 1], tok.dt[t0:t1, b:b + 1])


def _cat(*streams):
    return tuple(np.concatenate([s[i] for s in streams]) for i in range(4))


def _brute(work, b, stream):
    """Brute-force outputs [steps][nheads][headdim] and final state of sequence b."""
    x, B, C, dt = (np.asarray(a, np.float64) for a in stream)
    h0 = work.h0[b:b + 1].astype(np.float64)
    if x.shape[0] == 0:
        return np.zeros((0,) + work.h0.shape[1:3]), h0[0]
    y, H = brute_force(h0, x, B, C, dt, work.A.astype(np.float64), work.D.astype(np.float64))
    return y[:, 0], H[0]


def _models(work, b):
    """One ReplayModel per head of sequence b, with its n0[b] records committed."""
    sh = work.shape
    models = [forms.ReplayModel(work.h0[b, h], work.A[h], work.D[h], sh.window) for h in range(sh.nheads)]
    hpg = sh.nheads // sh.ngroups
    for t in range(int(work.n0[b])):
        for h, m in enumerate(models):
            g = h // hpg
            m.decode(work.pre.x[t, b, h], work.pre.B[t, b, g], work.pre.C[t, b, g], work.pre.dt[t, b, h])
    return models


def decode_work(in_dtype="f32"):
    return synth.decode_workload(SHAPE, 11, seed=4100 + (in_dtype == "bf16"), in_dtype=in_dtype,
                                 n0=np.array([0, 3, 1, 2], np.int32))


def verify_work(in_dtype="f32"):
    # one more round of tokens than the pins use, so a mis-sliced draft window
    # still finds tokens and shows up as wrong values
    return synth.verify_workload(SHAPE, 9, 3, seed=4200 + (in_dtype == "bf16"), in_dtype=in_dtype,
                                 n0=np.array([2, 0, 3, 1], np.int32))


def pin_committed_state(om, orc):
    """The state after the n0[b] committed records: brute force over each
    sequence's prefix, and the model's canonical state (checkpoint with the
    records folded)."""
    work = decode_work()
    H = om.committed_state(work, orc=orc)
    for b in range(SHAPE.batch):
        _, Hb = _brute(work, b, _stream(work.pre, 0, int(work.n0[b]), b))
        _close(H[b], Hb, f"committed state, sequence {b} vs brute force")
        for h, m in enumerate(_models(work, b)):
            _close(H[b, h], m.state(), f"committed state, sequence {b} head {h} vs replay model")
    seqs = np.array([3, 1])
    _close(om.committed_state(work, seqs=seqs, orc=orc), H[seqs], "committed state of selected sequences")


def pin_decode(om, orc):
    """Outputs of the first nsteps decode tokens and the state after them,
    against brute force over n0[b] records + those tokens, and against the
    model decoding them (folding every L records)."""
    for in_dtype in ("f32", "bf16"):
        work = decode_work(in_dtype)
        nsteps = 9
        y, H = om.decode(work, nsteps=nsteps, orc=orc)
        assert y.shape == (nsteps, SHAPE.batch, SHAPE.nheads, SHAPE.headdim), y.shape
        hpg = SHAPE.nheads // SHAPE.ngroups
        for b in range(SHAPE.batch):
            n0 = int(work.n0[b])
            yb, Hb = _brute(work, b, _cat(_stream(work.pre, 0, n0, b), _stream(work.steps, 0, nsteps, b)))
            _close(y[:, b], yb[n0:], f"decode outputs, sequence {b} vs brute force ({in_dtype})")
            _close(H[b], Hb, f"decode state, sequence {b} vs brute force ({in_dtype})")
            models = _models(work, b)
            for t in range(nsteps):
                for h, m in enumerate(models):
                    g = h // hpg
                    ym = m.decode(work.steps.x[t, b, h], work.steps.B[t, b, g], work.steps.C[t, b, g],
                                  work.steps.dt[t, b, h])
                    _close(y[t, b, h], ym, f"decode output t={t}, sequence {b} head {h} vs replay model")
            assert all(m.folds >= 2 for m in models), "the pin must cross several flushes"
        seqs = np.array([2, 0])
        ys, Hs = om.decode(work, nsteps=nsteps, seqs=seqs, orc=orc)
        _close(ys, y[:, seqs], "decode outputs of selected sequences")
        _close(Hs, H[seqs], "decode state of selected sequences")


def pin_verify_rounds(om, orc):
    """Draft outputs of every round and the state after the last commit,
    against brute force over each sequence's committed stream (n0[b] records,
    then the accepted prefix of every earlier round) + the round's drafts, and
    against the model verifying and committing round by round."""
    for in_dtype in ("f32", "bf16"):
        work = verify_work(in_dtype)
        T = work.extra["T"]
        acc = work.extra["accepted"]
        rounds = acc.shape[0] - 1
        y, H = om.verify_rounds(work, rounds=rounds, orc=orc)
        assert y.shape == (rounds, T, SHAPE.batch, SHAPE.nheads, SHAPE.headdim), y.shape
        assert len(set(acc[:rounds].ravel().tolist())) == T + 1, "acceptance must take every value 0..T"
        hpg = SHAPE.nheads // SHAPE.ngroups
        for b in range(SHAPE.batch):
            committed = _stream(work.pre, 0, int(work.n0[b]), b)
            models = _models(work, b)
            for r in range(rounds):
                drafts = _stream(work.steps, r * T, r * T + T, b)
                yb, _ = _brute(work, b, _cat(committed, drafts))
                _close(y[r, :, b], yb[-T:], f"round {r} drafts, sequence {b} vs brute force ({in_dtype})")
                a = int(acc[r, b])
                for h, m in enumerate(models):
                    g = h // hpg
                    ym = m.verify(work.steps.x[r * T:r * T + T, b, h], work.steps.B[r * T:r * T + T, b, g],
                                  work.steps.C[r * T:r * T + T, b, g], work.steps.dt[r * T:r * T + T, b, h])
                    _close(y[r, :, b, h], ym, f"round {r} drafts, sequence {b} head {h} vs replay model")
                    m.commit(a)
                committed = _cat(committed, tuple(d[:a] for d in drafts))
            _, Hb = _brute(work, b, committed)
            _close(H[b], Hb, f"state after the last commit, sequence {b} vs brute force ({in_dtype})")
            for h, m in enumerate(models):
                _close(H[b, h], m.state(), f"state after the last commit, sequence {b} head {h} vs replay model")
            assert sum(m.folds for m in models) > 0, "the pin must cross a flush"
        seqs = np.array([3, 0])
        ys, Hs = om.verify_rounds(work, rounds=rounds, seqs=seqs, orc=orc)
        _close(ys, y[:, :, seqs], "draft outputs of selected sequences")
        _close(Hs, H[seqs], "state of selected sequences")


ALL_PINS = [pin_committed_state, pin_decode, pin_verify_rounds]
