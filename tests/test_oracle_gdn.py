"""The fp64 GDN oracle against its pins, planted mistakes against the pins, and
the replay form (checkpoint + corrected-value records) against the definition."""
import types
from pathlib import Path

import numpy as np
import pytest

from oracle import gdn
from tests import gdn_pins

SRC = (Path(__file__).resolve().parent.parent / "oracle" / "gdn.py").read_text()


@pytest.mark.parametrize("pin", gdn_pins.PINS, ids=lambda p: p.__name__)
def test_gdn_pin(pin):
    pin(gdn)


def test_gdn_pin_mamba2(orc):
    gdn_pins.pin_orthonormal_keys_are_mamba2(gdn, orc)


MUTANTS = {
    "correction_sign": ("(eye - bt[..., None, None]", "(eye + bt[..., None, None]"),
    "no_decay": ("M = alpha[..., None, None] * (", "M = ("),
    "decay_sign": ("alpha = np.exp(np.asarray(g[t]", "alpha = np.exp(-np.asarray(g[t]"),
    "no_beta_on_value": ("+ bt[..., None, None] * vt[..., :, None]", "+ vt[..., :, None]"),
    "no_beta_on_correction": ("(eye - bt[..., None, None] * kt", "(eye - kt"),
    "left_multiply": ("np.matmul(S[act], M)", "np.matmul(M, S[act])"),
    "outer_transposed": ("vt[..., :, None] * kt[..., None, :]", "kt[..., :, None] * vt[..., None, :]"),
    "read_with_key": ("np.matmul(S[act], qt[..., :, None])", "np.matmul(S[act], kt[..., :, None])"),
    "wrong_head_map": ("return h // (nv // nk)", "return h % nk"),
    "decay_not_on_value": (
        "S[act] = np.matmul(S[act], M) + bt",
        "S[act] = np.matmul(S[act], M) + alpha[..., None, None] * bt"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not unique"
    mod = types.ModuleType(f"gdn_{name}")
    exec(compile(SRC.replace(old, new), f"gdn_{name}.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gdn_mutant_caught(name, orc):
    mod = _mutant(name)
    caught = []
    for pin in gdn_pins.PINS:
        try:
            pin(mod)
        except Exception:
            caught.append(pin.__name__)
    try:
        gdn_pins.pin_orthonormal_keys_are_mamba2(mod, orc)
    except Exception:
        caught.append("pin_orthonormal_keys_are_mamba2")
    assert caught, f"mutant {name} passed every pin"


def _workload(seed, steps=14, batch=2, nv=4, nk=2, dk=8, dv=6):
    r = np.random.Generator(np.random.PCG64(seed))
    q, k, v, g, beta = gdn_pins._tokens(r, steps, batch, nv, nk, dk, dv)
    S0 = 0.1 * r.standard_normal((batch, nv, dv, dk))
    return S0, q, k, v, g, beta


@pytest.mark.parametrize("window", [1, 2, 3, 5, 16])
def test_replay_form_equals_stepping(window):
    """Checkpoint + records with flush-at-start reproduce the stepped outputs
    and, after folding what is left, the stepped state (fp64, 1e-10)."""
    S0, q, k, v, g, beta = _workload(11 + window)
    S, o = gdn.conventional(S0, q, k, v, g, beta)
    S2, o2 = gdn.replay_decode(S0, q, k, v, g, beta, window)
    assert np.abs(o - o2).max() <= 1e-10 * np.abs(o).max()
    assert np.abs(S - S2).max() <= 1e-10 * np.abs(S).max()


def test_replay_rollback_equals_accepted_prefix():
    """Verify T drafts, commit a, keep decoding: equals stepping only the
    accepted drafts (the outputs of drafts 0..a-1 are those of stepping)."""
    S0, q, k, v, g, beta = _workload(21, steps=3 * 6)
    T, batch, nv = 3, S0.shape[0], S0.shape[1]
    r = np.random.Generator(np.random.PCG64(22))
    acc = r.integers(0, T + 1, size=(6, batch))
    rep = gdn.Replay(S0, nv, q.shape[2])
    kept = [[] for _ in range(batch)]
    for rd in range(6):
        for b in range(batch):
            if len(rep.records[b]) >= 4:
                rep.fold(b)
            drafts = [(q[rd * T + i, b], k[rd * T + i, b], v[rd * T + i, b], g[rd * T + i, b],
                       beta[rd * T + i, b]) for i in range(T)]
            outs, recs = rep.verify(b, drafts)
            # every draft's output equals stepping the kept tokens, then drafts 0..i
            for i in range(T):
                idx = kept[b] + [rd * T + j for j in range(i + 1)]
                sl = np.array(idx)
                _, oref = gdn.conventional(S0[b:b + 1], q[sl, b:b + 1], k[sl, b:b + 1], v[sl, b:b + 1],
                                           g[sl, b:b + 1], beta[sl, b:b + 1])
                assert np.abs(outs[i] - oref[-1, 0]).max() <= 1e-10 * np.abs(oref[-1, 0]).max()
            rep.commit(b, recs, int(acc[rd, b]))
            kept[b] += [rd * T + j for j in range(int(acc[rd, b]))]
    for b in range(batch):
        rep.fold(b)
        sl = np.array(kept[b], dtype=int)
        Sref, _ = gdn.conventional(S0[b:b + 1], q[sl, b:b + 1], k[sl, b:b + 1], v[sl, b:b + 1],
                                   g[sl, b:b + 1], beta[sl, b:b + 1])
        assert np.abs(rep.ckpt[b] - Sref[0]).max() <= 1e-10 * np.abs(Sref).max()
