"""GPU parity of the Gated DeltaNet layer at the edges the library accepts.

* Windows of one and two records (NVIDIA Developer blog "ReplaySSM: Rethinking
  State Storage for Faster Hybrid-Model Decoding", section "How ReplaySSM
  represents the state": a flush happens when the buffer of L records fills;
  with L = 1 every call that finds a record folds it first), for decode and for
  verification with T = 3 drafts.
* Degenerate gate and input values that the oracle's pins fix: beta = 0 (the
  delta rule writes nothing and the state only decays by exp of the summed
  gates), g = 0 (alpha = 1: no decay), q = 0 (every output exactly zero: the
  tile product, the key-query scores and the drafts' own terms all vanish),
  and gates strong enough that exp of a window's summed gates underflows fp32
  inside the window.
Each against the fp64 definition (oracle/gdn.py), outputs per row and the
state after a final flush per head.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from mamba_state_replay_amd import synth_gdn as sg
from tests.gpu_util import TOL, assert_rows_close, say

pytestmark = pytest.mark.gpu

LAYER = dict(nv=32, nk=16, dk=128, dv=128)
TINY = dict(nv=4, nk=2, dk=16, dv=32)


def _bg():
    from mamba_state_replay_amd import binding_gdn as bg
    return bg


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _state_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref).max(axis=(-1, -2)) / np.maximum(np.abs(ref).max(axis=(-1, -2)), 1e-30)


def _run(w, T, rounds):
    """Decode (T = None) or verify + commit rounds, then a flush; returns the
    outputs as [rounds][T][batch][nv][dv] (T = 1 for decode) and the state."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    dev = _dev()
    shape = w.shape
    TT = T or 1
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, TT, "bf16")
    st = bg.GdnState.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(np.ascontiguousarray(w.S0)).to(dev))
    ts = GdnTokenStream(w.steps, dev, TT)
    o = torch.empty((rounds, shape.batch, TT, shape.nv, shape.dv), device=dev)
    if T is None:
        for t in range(rounds):
            bg.gdn_decode_step(cfg, st, ts.call(t), o[t])
    else:
        acc = torch.from_numpy(w.extra["accepted"]).to(dev)
        for r in range(rounds):
            bg.gdn_verify_drafts(cfg, st, ts.call(r), o[r])
            bg.gdn_commit(cfg, st, acc[r], T)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    assert int(st.status.cpu()[0]) == 0
    return np.swapaxes(o.cpu().numpy(), 1, 2), st.ckpt.cpu().numpy()


def _reference(w, T, rounds):
    """The definition stepped token by token: all drafts' outputs of a round
    from the committed state, then the accepted prefix committed."""
    tk = w.steps
    S = w.S0.astype(np.float64)
    TT = T or 1
    oref = np.zeros((rounds, TT, w.shape.batch, w.shape.nv, w.shape.dv))
    for r in range(rounds):
        sl = slice(r * TT, (r + 1) * TT)
        args = (tk.q[sl], tk.k[sl], tk.v[sl], tk.g[sl], tk.beta[sl])
        if T is None:
            S, oref[r] = ogdn.conventional(S, *args)
        else:
            _, oref[r] = ogdn.conventional(S, *args)
            S, _ = ogdn.conventional(S, *args, nsteps=w.extra["accepted"][r])
    return oref, S


@pytest.mark.parametrize("L", [1, 2])
@pytest.mark.parametrize("T", [None, 3], ids=["decode", "verify3"])
def test_gdn_short_windows(L, T):
    shape = sg.GdnShape(batch=3, window=L, max_drafts=T or 1, **LAYER)
    rounds = 13 if T is None else 10
    w = sg.gdn_workload(shape, rounds, 3101 + L, "bf16", T=T)
    say(f"gdn {'decode' if T is None else f'verify T={T}'} L={L} cap={shape.cap}, {rounds} calls")
    y, S = _run(w, T, rounds)
    yref, Sref = _reference(w, T, rounds)
    assert_rows_close(y, yref, what=f"gdn outputs L={L}")
    assert _state_err(S, Sref).max() <= TOL


def _degenerate(w, case):
    tk = w.steps
    if case == "beta0":
        return dataclasses.replace(w, steps=dataclasses.replace(tk, beta=np.zeros_like(tk.beta)))
    if case == "g0":
        return dataclasses.replace(w, steps=dataclasses.replace(tk, g=np.zeros_like(tk.g)))
    if case == "q0":
        kw = dict(q=np.zeros_like(tk.q))
        if tk.q_bits is not None:
            kw["q_bits"] = np.zeros_like(tk.q_bits)
        return dataclasses.replace(w, steps=dataclasses.replace(tk, **kw))
    if case == "strong_decay":
        # even value heads: g in [-60, -40) per token, so exp of the gates over two
        # tokens (below e^-80) underflows fp32 inside every window
        g = tk.g.copy()
        r = np.random.default_rng(3121)
        g[..., 0::2] = (-40.0 - 20.0 * r.random(g[..., 0::2].shape)).astype(np.float32)
        return dataclasses.replace(w, steps=dataclasses.replace(tk, g=g))
    raise ValueError(case)


@pytest.mark.parametrize("case", ["beta0", "g0", "q0", "strong_decay"])
@pytest.mark.parametrize("T", [None, 3], ids=["decode", "verify3"])
@pytest.mark.parametrize("dims", ["layer", "tiny"])
def test_gdn_degenerate_inputs(case, T, dims):
    shape = sg.GdnShape(batch=3, window=4, max_drafts=T or 1, **(LAYER if dims == "layer" else TINY))
    rounds = 11 if T is None else 8
    w = _degenerate(sg.gdn_workload(shape, rounds, 3111, "bf16", T=T), case)
    say(f"gdn {dims} {'decode' if T is None else f'verify T={T}'} with {case}, {rounds} calls")
    y, S = _run(w, T, rounds)
    yref, Sref = _reference(w, T, rounds)
    assert_rows_close(y, yref, what=f"gdn outputs ({case})")
    assert _state_err(S, Sref).max() <= TOL
    if case == "q0":
        assert np.array_equal(y, np.zeros_like(y)), "q = 0: the outputs are not exactly zero"
    if case == "beta0" and T is None:
        # nothing is written: the state is the start decayed by each head's summed gates
        decay = np.exp(w.steps.g[:rounds].astype(np.float64).sum(axis=0))        # [batch][nv]
        want = w.S0.astype(np.float64) * decay[:, :, None, None]
        assert _state_err(S, want).max() <= TOL
