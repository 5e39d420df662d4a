"""Checks that pin the fp64 oracle to facts outside itself.

Each check takes a loaded oracle build and raises AssertionError when the
oracle disagrees with a closed form, a textbook/library routine, a brute-force
evaluation or the hand-worked example.  test_oracle_pins.py runs them on the
real oracle; test_oracle_mutations.py runs them on oracle builds with a
planted mistake and expects at least one to fail.

The recurrence being pinned is the Mamba-2 decode step (NVIDIA Developer blog
"ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding",
section "Why SSM layers can become a decoding bottleneck").
"""
from __future__ import annotations

import json
from pathlib import Path

import numpy as np
import scipy.signal

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rand_inputs(g, steps, batch, nh, hd, ds, ng):
    x = g.standard_normal((steps, batch, nh, hd))
    B = g.standard_normal((steps, batch, ng, ds))
    C = g.standard_normal((steps, batch, ng, ds))
    dt = np.logaddexp(0.0, g.standard_normal((steps, batch, nh)) - 2.0)
    A = -np.exp(g.uniform(0.0, np.log(16.0), nh))
    D = g.standard_normal(nh)
    return x, B, C, dt, A, D


def brute_force(h0, x, B, C, dt, A, D):
    """Unrolled closed form, no recurrence.

    H_t = (prod_{i<=t} e^{dt_i A}) H_0 + sum_{k<=t} (prod_{k<i<=t} e^{dt_i A}) dt_k x_k B_k^T
    y_t = H_t C_t + D x_t.  Decay products are products of per-step factors.
    """
    steps, batch, nh, hd = x.shape
    ng = B.shape[2]
    hpg = nh // ng
    y = np.zeros_like(x)
    Hs = np.zeros(h0.shape)
    for b in range(batch):
        for h in range(nh):
            g = h // hpg
            fac = np.exp(dt[:, b, h] * A[h])
            for t in range(steps):
                H = np.prod(fac[: t + 1]) * h0[b, h]
                for k in range(t + 1):
                    H = H + np.prod(fac[k + 1: t + 1]) * dt[k, b, h] * np.outer(x[k, b, h], B[k, b, g])
                y[t, b, h] = H @ C[t, b, g] + D[h] * x[t, b, h]
                if t == steps - 1:
                    Hs[b, h] = H
    return y, Hs


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) / scale if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: normalized error {err:.3e} > {tol:.1e}"


def pin_brute_force_tiny(orc):
    """Tiny workload shape (batch 1, 4 heads, 16x16 tiles, 1 group), 64 steps."""
    g = np.random.default_rng(11)
    x, B, C, dt, A, D = _rand_inputs(g, 64, 1, 4, 16, 16, 1)
    h0 = g.standard_normal((1, 4, 16, 16)) * 0.1
    H, y = orc.conventional(h0, x, B, C, dt, A, D)
    yb, Hb = brute_force(h0, x, B, C, dt, A, D)
    _close(y, yb, 1e-12, "outputs vs brute force")
    _close(H, Hb, 1e-12, "state vs brute force")


def pin_brute_force_groups(orc):
    """Non-square tiles and two groups (heads 0,1 -> group 0; 2,3 -> group 1)."""
    g = np.random.default_rng(12)
    x, B, C, dt, A, D = _rand_inputs(g, 12, 2, 4, 5, 7, 2)
    h0 = g.standard_normal((2, 4, 5, 7))
    H, y = orc.conventional(h0, x, B, C, dt, A, D)
    yb, Hb = brute_force(h0, x, B, C, dt, A, D)
    _close(y, yb, 1e-12, "outputs vs brute force (groups)")
    _close(H, Hb, 1e-12, "state vs brute force (groups)")


def pin_eq_z_single_update(orc):
    """One update from a zero state: (dt x B^T) C = dt (B.C) x (section
    "Benefit 2": the left side builds a state and reads it, the right side
    scales a vector by a scalar)."""
    g = np.random.default_rng(13)
    x, B, C, dt, A, D = _rand_inputs(g, 1, 3, 4, 6, 9, 2)
    h0 = np.zeros((3, 4, 6, 9))
    _, y = orc.conventional(h0, x, B, C, dt, A, D)
    for b in range(3):
        for h in range(4):
            gi = h // 2
            expect = dt[0, b, h] * float(B[0, b, gi] @ C[0, b, gi]) * x[0, b, h] + D[h] * x[0, b, h]
            _close(y[0, b, h], expect, 1e-13, "Eq.Z single update")


def pin_no_decay_is_sum(orc):
    """A = 0: no decay, the state is the plain sum of the rank-1 inputs.
    Small integers make every value exact."""
    g = np.random.default_rng(14)
    steps, nh, hd, ds = 6, 2, 3, 4
    x = g.integers(-3, 4, (steps, 1, nh, hd)).astype(float)
    B = g.integers(-3, 4, (steps, 1, 1, ds)).astype(float)
    C = g.integers(-3, 4, (steps, 1, 1, ds)).astype(float)
    dt = g.integers(1, 3, (steps, 1, nh)).astype(float)
    h0 = g.integers(-2, 3, (1, nh, hd, ds)).astype(float)
    A = np.zeros(nh)
    D = np.array([2.0, -1.0])
    H, y = orc.conventional(h0, x, B, C, dt, A, D)
    acc = h0[0].copy()
    for t in range(steps):
        for h in range(nh):
            acc[h] += dt[t, 0, h] * np.outer(x[t, 0, h], B[t, 0, 0])
            expect = acc[h] @ C[t, 0, 0] + D[h] * x[t, 0, h]
            assert np.array_equal(y[t, 0, h], expect), "A=0 outputs are not the exact sum"
    assert np.array_equal(H[0], acc), "A=0 state is not the exact sum"


def pin_dt_zero_keeps_state(orc):
    """dt = 0: decay exp(0) = 1 and no input, so H stays H0 and y = H0 C + D x."""
    g = np.random.default_rng(15)
    x, B, C, dt, A, D = _rand_inputs(g, 5, 2, 2, 4, 3, 1)
    dt[:] = 0.0
    h0 = g.standard_normal((2, 2, 4, 3))
    H, y = orc.conventional(h0, x, B, C, dt, A, D)
    assert np.array_equal(H, h0), "dt=0 changed the state"
    for t in range(5):
        for b in range(2):
            for h in range(2):
                _close(y[t, b, h], h0[b, h] @ C[t, b, 0] + D[h] * x[t, b, h], 1e-14, "dt=0 output")


def pin_c_zero_is_skip(orc):
    """C = 0: the state read vanishes and y = D x exactly."""
    g = np.random.default_rng(16)
    x, B, C, dt, A, D = _rand_inputs(g, 7, 1, 3, 4, 5, 1)
    C[:] = 0.0
    h0 = g.standard_normal((1, 3, 4, 5))
    _, y = orc.conventional(h0, x, B, C, dt, A, D)
    assert np.array_equal(y, D[None, None, :, None] * x), "C=0 output is not D x"


def pin_scalar_geometric(orc):
    """1x1 state, constant dt and A, x = B = 1: h_t = a^t h0 + dt (1 - a^t)/(1 - a),
    the geometric series with ratio a = exp(dt A) < 1."""
    steps, dtv, Av, h0v = 40, 0.3, -2.5, 0.7
    a = np.exp(dtv * Av)
    x = np.ones((steps, 1, 1, 1))
    B = np.ones((steps, 1, 1, 1))
    C = np.ones((steps, 1, 1, 1))
    dt = np.full((steps, 1, 1), dtv)
    H, y = orc.conventional(np.full((1, 1, 1, 1), h0v), x, B, C, dt, np.array([Av]), np.array([0.0]))
    t = np.arange(1, steps + 1)
    expect = a ** t * h0v + dtv * (1 - a ** t) / (1 - a)
    _close(y[:, 0, 0, 0], expect, 1e-13, "geometric closed form")


def pin_scalar_lfilter(orc):
    """1x1 state with constant decay is the first-order IIR filter
    h_t = a h_{t-1} + u_t, u_t = dt x_t B_t; scipy.signal.lfilter computes it."""
    g = np.random.default_rng(17)
    steps, dtv, Av = 50, 0.2, -1.7
    a = np.exp(dtv * Av)
    x = g.standard_normal((steps, 1, 1, 1))
    B = g.standard_normal((steps, 1, 1, 1))
    C = g.standard_normal((steps, 1, 1, 1))
    dt = np.full((steps, 1, 1), dtv)
    D = np.array([0.4])
    h0 = 1.3
    H, y = orc.conventional(np.full((1, 1, 1, 1), h0), x, B, C, dt, np.array([Av]), D)
    u = dtv * x[:, 0, 0, 0] * B[:, 0, 0, 0]
    h, _ = scipy.signal.lfilter([1.0], [1.0, -a], u, zi=[a * h0])
    expect = h * C[:, 0, 0, 0] + D[0] * x[:, 0, 0, 0]
    _close(y[:, 0, 0, 0], expect, 1e-12, "lfilter")
    _close(H[0, 0, 0, 0], h[-1], 1e-12, "lfilter final state")


def pin_group_mapping(orc):
    """4 heads, 2 groups: heads 0,1 read group 0, heads 2,3 read group 1.
    With B of group 1 set to zero, heads 2,3 only decay."""
    g = np.random.default_rng(18)
    x, B, C, dt, A, D = _rand_inputs(g, 9, 1, 4, 3, 4, 2)
    B[:, :, 1] = 0.0
    h0 = g.standard_normal((1, 4, 3, 4))
    H, _ = orc.conventional(h0, x, B, C, dt, A, D)
    for h in (2, 3):
        decay = np.prod(np.exp(dt[:, 0, h] * A[h]))
        _close(H[0, h], decay * h0[0, h], 1e-13, f"head {h} should only decay")
    for h in (0, 1):
        decay = np.prod(np.exp(dt[:, 0, h] * A[h]))
        assert np.max(np.abs(H[0, h] - decay * h0[0, h])) > 1e-3, f"head {h} got no input"


def pin_worked_example(orc):
    """Hand-derived two-step example (tests/golden/two_step_worked_example.json)."""
    ex = json.loads((GOLDEN / "two_step_worked_example.json").read_text())
    arr = {k: np.array(ex[k], float) for k in ("A", "D", "dt", "x", "B", "C", "expected_y", "expected_H")}
    h0 = np.zeros(arr["expected_H"].shape)
    H, y = orc.conventional(h0, arr["x"], arr["B"], arr["C"], arr["dt"], arr["A"], arr["D"])
    _close(y, arr["expected_y"], ex["tolerance"], "worked example outputs")
    _close(H, arr["expected_H"], ex["tolerance"], "worked example state")


def pin_partial_steps(orc):
    """nsteps[b] tokens per sequence equal a separate run over that prefix."""
    g = np.random.default_rng(19)
    x, B, C, dt, A, D = _rand_inputs(g, 6, 3, 2, 3, 4, 1)
    h0 = g.standard_normal((3, 2, 3, 4))
    ns = np.array([0, 4, 6], np.int32)
    H, _ = orc.conventional(h0, x, B, C, dt, A, D, nsteps=ns)
    for b in range(3):
        n = ns[b]
        Hb, _ = orc.conventional(h0[b:b + 1], x[:n, b:b + 1], B[:n, b:b + 1], C[:n, b:b + 1],
                                 dt[:n, b:b + 1], A, D)
        assert np.array_equal(H[b], Hb[0]), "per-sequence step counts differ from a prefix run"
    assert np.array_equal(H[0], h0[0])


ALL_PINS = [
    pin_brute_force_tiny,
    pin_brute_force_groups,
    pin_eq_z_single_update,
    pin_no_decay_is_sum,
    pin_dt_zero_keeps_state,
    pin_c_zero_is_skip,
    pin_scalar_geometric,
    pin_scalar_lfilter,
    pin_group_mapping,
    pin_worked_example,
    pin_partial_steps,
]
