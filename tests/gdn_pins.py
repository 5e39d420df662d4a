"""Pins of the fp64 GDN oracle (oracle/gdn.py) against facts fixed outside it.

Each pin takes the oracle module (so that planted mistakes in a copy of it can
be run through the same pins) and raises AssertionError on a mismatch.  The
facts are those of the gated delta rule (Yang, Kautz and Hatamizadeh, "Gated
Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025) and of the
ReplaySSM page's statement that GDN's update keeps Mamba-2's decay-plus-rank-1
structure (NVIDIA Developer blog "ReplaySSM ...", section "Why SSM layers can
become a decoding bottleneck"):

* delta-rule write: with no decay, beta = 1 and a unit key, the state maps the
  key exactly to the value (S_t k_t = v_t) and leaves every direction
  orthogonal to the key unchanged;
* beta = 0: the state only decays, by exp(sum g);
* orthonormal keys from a zero state: no correction term ever acts, so the
  layer is the Mamba-2 recurrence with x = v, B = k, C = q, dt = beta and
  decay exp(g); checked against the (separately pinned) Mamba-2 C oracle;
* a 1 x 1 state with constant inputs: the geometric series closed form;
* brute force: the unrolled product of the per-step transition matrices;
* the value-to-key head map in contiguous blocks.
"""
from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _tokens(r, steps, batch, nv, nk, dk, dv):
    q = r.standard_normal((steps, batch, nk, dk))
    k = _unit(r.standard_normal((steps, batch, nk, dk)))
    v = r.standard_normal((steps, batch, nv, dv))
    g = -r.uniform(0.01, 1.0, (steps, batch, nv))
    beta = r.uniform(0.05, 0.95, (steps, batch, nv))
    return q, k, v, g, beta


def pin_delta_write(mod):
    """g = 0, beta = 1, unit k: S_t k = v and S_t x = S_{t-1} x for x orthogonal to k."""
    r = _rng(1)
    batch, nv, nk, dk, dv = 2, 4, 2, 8, 6
    S0 = r.standard_normal((batch, nv, dv, dk))
    q, k, v, g, beta = _tokens(r, 1, batch, nv, nk, dk, dv)
    g[:] = 0.0
    beta[:] = 1.0
    q[:] = k                                    # read back along the key
    S1, o = mod.conventional(S0, q, k, v, g, beta)
    assert np.allclose(o[0], v[0], atol=1e-12, rtol=0), "S_t k_t != v_t"
    for b in range(batch):
        for h in range(nv):
            kv = k[0, b, h // (nv // nk)]
            x = r.standard_normal(dk)
            x -= kv * (kv @ x)                  # orthogonal to the key
            assert np.allclose(S1[b, h] @ x, S0[b, h] @ x, atol=1e-12, rtol=0)


def pin_beta_zero(mod):
    """beta = 0: S_t = exp(sum g) S_0 and o_t = S_t q_t."""
    r = _rng(2)
    batch, nv, nk, dk, dv, steps = 2, 4, 1, 5, 7, 6
    S0 = r.standard_normal((batch, nv, dv, dk))
    q, k, v, g, beta = _tokens(r, steps, batch, nv, nk, dk, dv)
    beta[:] = 0.0
    S, o = mod.conventional(S0, q, k, v, g, beta)
    G = np.exp(np.cumsum(g, axis=0))            # [steps][batch][nv]
    assert np.allclose(S, G[-1][..., None, None] * S0, atol=1e-13, rtol=1e-12)
    for t in range(steps):
        ref = G[t][..., None] * np.einsum("bhij,bj->bhi", S0, q[t][:, 0])
        assert np.allclose(o[t], ref, atol=1e-12, rtol=1e-12)


def pin_orthonormal_keys_are_mamba2(mod, orc):
    """Orthonormal keys from S_0 = 0: equals the Mamba-2 recurrence (x=v, B=k,
    C=q, dt=beta, A*dt=g) of the C oracle, with D = 0."""
    r = _rng(3)
    batch, nv, nk, dk, dv, steps = 2, 6, 3, 8, 5, 8
    q, k, v, g, beta = _tokens(r, steps, batch, nv, nk, dk, dv)
    for b in range(batch):
        for kh in range(nk):
            Q, _ = np.linalg.qr(r.standard_normal((dk, dk)))
            k[:, b, kh] = Q[:, :steps].T        # step t uses column t: orthonormal over time
    A = -r.uniform(0.2, 2.0, nv)
    dt = beta.copy()
    g = dt * A[None, None, :]
    S0 = np.zeros((batch, nv, dv, dk))
    S, o = mod.conventional(S0, q, k, v, g, beta)
    H, y = orc.conventional(S0, v, k, q, dt, A, np.zeros(nv))
    assert np.allclose(S, H, atol=1e-12, rtol=1e-11), "state differs from the Mamba-2 recurrence"
    assert np.allclose(o, y, atol=1e-12, rtol=1e-11), "outputs differ from the Mamba-2 recurrence"


def pin_scalar_geometric(mod):
    """dk = dv = 1, constant inputs: s_t = r^t s_0 + c (1 - r^t) / (1 - r),
    r = alpha (1 - beta k^2), c = beta v k; o_t = s_t q."""
    steps = 12
    alpha, beta, kv, vv, qv, s0 = 0.8, 0.3, 0.6, 1.7, -0.9, 0.4
    q = np.full((steps, 1, 1, 1), qv)
    k = np.full((steps, 1, 1, 1), kv)
    v = np.full((steps, 1, 1, 1), vv)
    g = np.full((steps, 1, 1), np.log(alpha))
    b = np.full((steps, 1, 1), beta)
    S, o = mod.conventional(np.full((1, 1, 1, 1), s0), q, k, v, g, b)
    rr, c = alpha * (1 - beta * kv * kv), beta * vv * kv
    t = np.arange(1, steps + 1)
    ref = rr ** t * s0 + c * (1 - rr ** t) / (1 - rr)
    assert np.allclose(o[:, 0, 0, 0], ref * qv, atol=1e-14, rtol=1e-13)
    assert np.isclose(S[0, 0, 0, 0], ref[-1], atol=1e-14, rtol=1e-13)


def pin_unrolled_products(mod):
    """S_t = S_0 M_1 ... M_t + sum_j beta_j v_j k_j^T M_{j+1} ... M_t with
    M_i = alpha_i (I - beta_i k_i k_i^T), built from explicit matrix products."""
    r = _rng(5)
    batch, nv, nk, dk, dv, steps = 1, 2, 2, 4, 3, 5
    S0 = r.standard_normal((batch, nv, dv, dk))
    q, k, v, g, beta = _tokens(r, steps, batch, nv, nk, dk, dv)
    S, o = mod.conventional(S0, q, k, v, g, beta)
    for h in range(nv):
        kh = h // (nv // nk)
        Ms = [np.exp(g[i, 0, h]) * (np.eye(dk) - beta[i, 0, h] * np.outer(k[i, 0, kh], k[i, 0, kh]))
              for i in range(steps)]
        for t in range(steps):
            acc = S0[0, h] @ np.linalg.multi_dot([np.eye(dk)] + Ms[:t + 1])
            for j in range(t + 1):
                tail = np.linalg.multi_dot([np.eye(dk), np.eye(dk)] + Ms[j + 1:t + 1])
                acc = acc + beta[j, 0, h] * np.outer(v[j, 0, h], k[j, 0, kh]) @ tail
            assert np.allclose(o[t, 0, h], acc @ q[t, 0, kh], atol=1e-12, rtol=1e-11)
        assert np.allclose(S[0, h], acc, atol=1e-12, rtol=1e-11)


def pin_head_map(mod):
    """Zeroing key head 0 (and its keys' queries) leaves only value heads
    0 .. nv/nk - 1 reading zeros: value heads map to key heads in blocks."""
    r = _rng(6)
    batch, nv, nk, dk, dv = 1, 6, 3, 4, 4
    S0 = np.zeros((batch, nv, dv, dk))
    q, k, v, g, beta = _tokens(r, 1, batch, nv, nk, dk, dv)
    q[:, :, 0] = 0.0
    _, o = mod.conventional(S0, q, k, v, g, beta)
    per = nv // nk
    assert np.all(o[0, 0, :per] == 0.0)
    assert np.all(np.abs(o[0, 0, per:]).max(axis=-1) > 0)
    assert mod.key_head(per, nv, nk) == 1 and mod.key_head(per - 1, nv, nk) == 0


def pin_nsteps(mod):
    """Per-sequence step counts equal separate prefix runs."""
    r = _rng(7)
    batch, nv, nk, dk, dv, steps = 3, 2, 1, 4, 4, 5
    S0 = r.standard_normal((batch, nv, dv, dk))
    q, k, v, g, beta = _tokens(r, steps, batch, nv, nk, dk, dv)
    n = np.array([0, 2, 5])
    S, o = mod.conventional(S0, q, k, v, g, beta, nsteps=n)
    for b in range(batch):
        sl = slice(b, b + 1)
        Sb, ob = mod.conventional(S0[sl], q[:n[b], sl], k[:n[b], sl], v[:n[b], sl], g[:n[b], sl],
                                  beta[:n[b], sl])
        assert np.array_equal(S[b], Sb[0])
        assert np.array_equal(o[:n[b], b], ob[:, 0])
        assert np.all(np.isnan(o[n[b]:, b]))


PINS = [pin_delta_write, pin_beta_zero, pin_scalar_geometric, pin_unrolled_products, pin_head_map,
        pin_nsteps]
PINS_WITH_MAMBA2 = [pin_orthonormal_keys_are_mamba2]
