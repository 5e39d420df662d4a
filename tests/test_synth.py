"""The seeded input generator: determinism, shapes, laws and bf16 rounding."""
import numpy as np
import torch

from mamba_state_replay_amd import synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, 65504.0], np.float32),
                        # exact halfway cases between neighbouring bf16 values
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    bits = synth.bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = synth.bf16_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_deterministic_and_shaped():
    shape = synth.LayerShape(batch=3, nheads=8, headdim=4, dstate=6, ngroups=2, window=4)
    w1 = synth.decode_workload(shape, 5, seed=1001, n0=4)
    w2 = synth.decode_workload(shape, 5, seed=1001, n0=4)
    for a, b in [(w1.h0, w2.h0), (w1.steps.x, w2.steps.x), (w1.steps.dt, w2.steps.dt), (w1.A, w2.A)]:
        assert np.array_equal(a, b)
    assert w1.steps.x.shape == (5, 3, 8, 4)
    assert w1.steps.B.shape == (5, 3, 2, 6)
    assert w1.steps.dt.shape == (5, 3, 8)
    assert w1.pre.steps == 4
    assert w1.steps.x_bits.dtype == np.uint16
    assert np.array_equal(synth.bf16_to_f32(w1.steps.x_bits), w1.steps.x)
    assert np.all(w1.A < 0) and np.all(w1.A >= -16.0001) and np.all(w1.A <= -1.0)
    assert np.all(w1.steps.dt > 0)


def test_laws_roughly():
    shape = synth.LayerShape(batch=64, nheads=16, headdim=16, dstate=32, ngroups=2)
    w = synth.decode_workload(shape, 4, seed=5, in_dtype="f32")
    assert abs(w.steps.x.mean()) < 0.02 and abs(w.steps.x.std() - 1) < 0.02
    assert abs(w.h0.std() - 0.1) < 0.002
    z = np.log(np.expm1(w.steps.dt.astype(np.float64)))   # inverse softplus
    assert abs(z.mean() + 2) < 0.05 and abs(z.std() - 1) < 0.05


def test_verify_workload_acceptance():
    shape = synth.LayerShape(batch=50, nheads=4, headdim=4, dstate=4, ngroups=1, window=16, max_drafts=3)
    w = synth.verify_workload(shape, rounds=10, T=3, seed=1003)
    acc = w.extra["accepted"]
    assert acc.shape == (10, 50) and acc.min() >= 0 and acc.max() <= 3
    assert set(np.unique(acc)) == {0, 1, 2, 3}
    assert w.steps.steps == 30
    assert np.all(w.n0 >= 0) and np.all(w.n0 < 16)


def test_gdn_tokens_shapes_and_laws():
    from mamba_state_replay_amd import synth_gdn as sg
    shape = sg.GdnShape(batch=3, nv=4, nk=2, dk=16, dv=32, window=4, max_drafts=2)
    w = sg.gdn_workload(shape, 5, seed=3)
    t = w.steps
    assert t.q.shape == (5, 3, 2, 16) and t.k.shape == (5, 3, 2, 16) and t.v.shape == (5, 3, 4, 32)
    assert t.g.shape == (5, 3, 4) and t.beta.shape == (5, 3, 4)
    # bf16 storage: values are the bf16 patterns widened
    assert np.array_equal((t.k_bits.astype(np.uint32) << 16).view(np.float32), t.k)
    # unit keys and queries of norm 1/sqrt(dk), up to bf16 rounding
    assert np.allclose(np.linalg.norm(t.k, axis=-1), 1.0, atol=1e-2)
    assert np.allclose(np.linalg.norm(t.q, axis=-1), 0.25, atol=1e-2)
    assert np.all(t.g < 0) and np.all((t.beta > 0) & (t.beta < 1))
    assert w.S0.shape == (3, 4, 32, 16)
    w2 = sg.gdn_workload(shape, 5, seed=3)
    assert np.array_equal(w2.steps.v, t.v) and np.array_equal(w2.S0, w.S0)
    v = sg.gdn_workload(shape, 4, seed=4, T=2)
    assert v.steps.steps == 8 and v.extra["accepted"].shape == (4, 3)
    assert v.extra["accepted"].min() >= 0 and v.extra["accepted"].max() <= 2
