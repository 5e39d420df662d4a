"""fp64 self-checks of the replay readings against the step-by-step definition.

* replay form == conventional outputs (the pages: the replayed outputs equal the
  stepped ones except for rounding)
* fold(checkpoint, records) == the stepped state
* output-only matrix form == replay form
* checkpoint + buffer driven by decode/verify/commit/flush == stepping only the
  committed tokens (rollback is a pointer move)
"""
import numpy as np
import pytest

from oracle import forms


def _tile_inputs(g, n, hd, ds):
    x = g.standard_normal((n, hd))
    B = g.standard_normal((n, ds))
    C = g.standard_normal((n, ds))
    dt = np.logaddexp(0.0, g.standard_normal(n) - 2.0)
    return x, B, C, dt


def _step(orc, H, x, B, C, dt, A, D):
    """Conventional oracle on one tile over n tokens: returns (H, y[n][hd])."""
    n, hd = x.shape
    ds = B.shape[1]
    Hn, y = orc.conventional(H[None, None], x[:, None, None], B[:, None, None], C[:, None, None],
                             dt[:, None, None], np.array([A]), np.array([D]))
    return Hn[0, 0], y[:, 0, 0]


@pytest.mark.parametrize("n,T", [(0, 1), (3, 1), (5, 3), (16, 1), (18, 3), (7, 8)])
def test_replay_and_output_only_match_conventional(orc, n, T):
    g = np.random.default_rng(100 + n * 10 + T)
    hd, ds = 6, 10
    Hs = g.standard_normal((hd, ds)) * 0.1
    A, D = -np.exp(g.uniform(0, np.log(16))), g.standard_normal()
    rx, rB, rC, rdt = _tile_inputs(g, n, hd, ds)
    qx, qB, qC, qdt = _tile_inputs(g, T, hd, ds)
    Hc, _ = _step(orc, Hs, rx, rB, rC, rdt, A, D)
    _, yc = _step(orc, Hc, qx, qB, qC, qdt, A, D)
    yr = forms.replay_outputs(Hs, rx, rB, rdt, A, D, qx, qB, qC, qdt)
    yo = forms.output_only(Hs, rx, rB, rdt, A, D, qx, qB, qC, qdt)
    scale = np.max(np.abs(yc))
    assert np.max(np.abs(yr - yc)) <= 1e-10 * scale
    assert np.max(np.abs(yo - yr)) <= 1e-10 * scale
    # fold == stepped state
    Hf = forms.replay_fold(Hs, rx, rB, rdt, A)
    assert np.max(np.abs(Hf - Hc)) <= 1e-10 * max(1.0, np.max(np.abs(Hc)))


def test_eq_z_output_only_single_query(orc):
    """Zero checkpoint, no records, one query: y = dt (B.C) x + D x."""
    g = np.random.default_rng(7)
    x, B, C, dt = _tile_inputs(g, 1, 5, 8)
    y = forms.output_only(np.zeros((5, 8)), x[:0], B[:0], dt[:0], -1.0, 0.3, x, B, C, dt)
    np.testing.assert_allclose(y[0], dt[0] * (B[0] @ C[0]) * x[0] + 0.3 * x[0], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("L", [1, 4, 16])
def test_replay_model_decode_equals_conventional(orc, L):
    g = np.random.default_rng(200 + L)
    hd, ds, steps = 4, 8, 40
    Hs = g.standard_normal((hd, ds)) * 0.1
    A, D = -np.exp(g.uniform(0, np.log(16))), g.standard_normal()
    x, B, C, dt = _tile_inputs(g, steps, hd, ds)
    _, yc = _step(orc, Hs, x, B, C, dt, A, D)
    m = forms.ReplayModel(Hs, A, D, L)
    for t in range(steps):
        y = m.decode(x[t], B[t], C[t], dt[t])
        assert np.max(np.abs(y - yc[t])) <= 1e-10 * max(1.0, np.max(np.abs(yc[t])))
        assert m.n <= L
    # fold at start: steps L+1, 2L+1, ... fold
    assert m.folds == (steps - 1) // L


def test_replay_model_rollback_equals_prefix_decode(orc):
    """verify(T) + commit(a) + more == stepping only the accepted drafts + more."""
    g = np.random.default_rng(300)
    hd, ds, T, L = 4, 6, 3, 5
    Hs = g.standard_normal((hd, ds)) * 0.1
    A, D = -np.exp(g.uniform(0, np.log(16))), g.standard_normal()
    m = forms.ReplayModel(Hs, A, D, L)
    H = Hs.copy()
    for r in range(25):
        qx, qB, qC, qdt = _tile_inputs(g, T, hd, ds)
        a = int(g.integers(0, T + 1))
        y = m.verify(qx, qB, qC, qdt)
        _, yc = _step(orc, H, qx, qB, qC, qdt, A, D)
        assert np.max(np.abs(y - yc)) <= 1e-10 * max(1.0, np.max(np.abs(yc)))
        m.commit(a)
        H, _ = _step(orc, H, qx[:a], qB[:a], qC[:a], qdt[:a], A, D)
        assert m.n <= L + T - 1
        assert np.max(np.abs(m.state() - H)) <= 1e-10 * max(1.0, np.max(np.abs(H)))
    m.flush()
    assert np.max(np.abs(m.Hs - H)) <= 1e-10 * max(1.0, np.max(np.abs(H)))
