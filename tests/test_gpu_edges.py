"""GPU parity at the edges the library accepts, and the device status contract.

* Windows of one and two records (NVIDIA Developer blog "ReplaySSM: Rethinking
  State Storage for Faster Hybrid-Model Decoding", section "How ReplaySSM
  represents the state": a flush happens when the buffer of L records fills;
  with L = 1 every call that finds a record flushes it), for decode and for
  verification with T = 3.
* Degenerate layer parameters that the oracle's pins fix exactly: A = 0 (no
  decay), dt = 0 (the state never moves), C = 0 (the output is D x, bit for
  bit), and a decay strong enough that exp of the window's segment sums
  underflows fp32 inside the window.
* Data errors the kernels find on the device: one head's copy of the ring
  pointer disagreeing with the others (a single non-zero head), and a ring
  overfilled by committing twice without a verification in between; each sets
  its status bit and NaNs only the affected outputs, and every other sequence's
  outputs are bit-identical to a clean run.
"""
import dataclasses

import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from tests.gpu_util import TOL, assert_rows_close, device, host, say, tile_err

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)


def _decode_run(cfg, work, steps, dev):
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps.slice(0, steps), dev)
    y = torch.empty((steps, cfg.batch, 1, cfg.nheads, cfg.headdim), device=dev)
    for t in range(steps):
        rb.replayssm_decode_step(cfg, st, p, stream.call(t), y[t])
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    return host(y)[:, :, 0], st


def _verify_run(cfg, work, T, dev):
    rounds = work.extra["accepted"].shape[0]
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, cfg.batch, T, cfg.nheads, cfg.headdim), device=dev)
    for r in range(rounds):
        rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
        rb.replayssm_commit(cfg, st, acc[r], T)
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    return np.swapaxes(host(y), 1, 2), st


@pytest.mark.parametrize("L", [1, 2])
def test_short_windows_decode(L):
    """Decode at L = 1 (ring of 2 slots: every call flushes the one committed
    record) and L = 2, from a full buffer, against the oracle; the final flush
    leaves the oracle's state."""
    dev = device()
    steps = 13
    shape = synth.LayerShape(batch=3, window=L, max_drafts=1, **NEMO)
    work = synth.decode_workload(shape, steps, seed=1101 + L, n0=L)
    cfg = staging.config(shape)
    say(f"decode L={L} cap={cfg.cap} {steps} steps")
    y, st = _decode_run(cfg, work, steps, dev)
    yref, Href = orc_mod.decode(work)
    assert_rows_close(y, yref, what=f"decode outputs L={L}")
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0


@pytest.mark.parametrize("L", [1, 2])
def test_short_windows_verify(L):
    """Verification with T = 3 drafts at L = 1 and L = 2 (ring of 2L + 5 slots):
    a round that starts with any committed record flushes them first, the drafts
    land past them, and rollback leaves only the accepted ones."""
    dev = device()
    T, rounds = 3, 12
    shape = synth.LayerShape(batch=4, window=L, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, rounds, T, seed=1111 + L)
    cfg = staging.config(shape)
    say(f"verify L={L} T={T} cap={cfg.cap} {rounds} rounds")
    y, st = _verify_run(cfg, work, T, dev)
    yref, Href = orc_mod.verify_rounds(work)
    assert_rows_close(y, yref, what=f"verify outputs L={L}")
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0


def _degenerate(work: synth.Workload, case: str) -> synth.Workload:
    """The workload with one parameter forced to its degenerate value (the
    stored input values change, bf16 bits included, so both sides see them)."""
    def tok_with(tok, **kw):
        return dataclasses.replace(tok, **kw)

    if case == "A0":
        return dataclasses.replace(work, A=np.zeros_like(work.A))
    if case == "dt0":
        return dataclasses.replace(work, pre=tok_with(work.pre, dt=np.zeros_like(work.pre.dt)),
                                   steps=tok_with(work.steps, dt=np.zeros_like(work.steps.dt)))
    if case == "C0":
        kw = dict(C=np.zeros_like(work.steps.C))
        if work.steps.C_bits is not None:
            kw["C_bits"] = np.zeros_like(work.steps.C_bits)
        return dataclasses.replace(work, steps=tok_with(work.steps, **kw))
    if case == "strong_decay":
        # even heads: A = -16 and dt in [2.5, 3.5), so a = dt A <= -40 per token and the
        # decay over three tokens, exp(-120), is below the smallest fp32 subnormal
        g = np.random.default_rng(1121)
        A = work.A.copy()
        A[0::2] = -16.0

        def strong(dt):
            dt = dt.copy()
            dt[..., 0::2] = (2.5 + g.random(dt[..., 0::2].shape)).astype(np.float32)
            return dt
        return dataclasses.replace(work, A=A, pre=tok_with(work.pre, dt=strong(work.pre.dt)),
                                   steps=tok_with(work.steps, dt=strong(work.steps.dt)))
    raise ValueError(case)


CASES = ["A0", "dt0", "C0", "strong_decay"]


@pytest.mark.parametrize("case", CASES)
def test_degenerate_parameters_decode(case):
    dev = device()
    L, steps = 4, 11
    shape = synth.LayerShape(batch=3, window=L, max_drafts=1, **NEMO)
    work = _degenerate(synth.decode_workload(shape, steps, seed=1131, n0=synth.staggered_fill(3, L)), case)
    cfg = staging.config(shape)
    say(f"decode with {case}, L={L}, {steps} steps")
    y, st = _decode_run(cfg, work, steps, dev)
    yref, Href = orc_mod.decode(work)
    assert_rows_close(y, yref, what=f"decode outputs ({case})")
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0
    if case == "C0":
        # H C = 0 and every record's score is 0, so the output is the one product D x
        want = work.D.astype(np.float32)[None, None, :, None] * work.steps.x[:steps].astype(np.float32)
        assert np.array_equal(y, want), "C = 0: the output is not exactly D x"
    if case == "dt0":
        # the state never moves: the flushed checkpoint is the initial one, bit for bit
        assert np.array_equal(host(st.ckpt), work.h0)


@pytest.mark.parametrize("case", CASES)
def test_degenerate_parameters_verify(case):
    dev = device()
    L, T, rounds = 4, 3, 9
    shape = synth.LayerShape(batch=4, window=L, max_drafts=T, **NEMO)
    work = _degenerate(synth.verify_workload(shape, rounds, T, seed=1141), case)
    cfg = staging.config(shape)
    say(f"verify with {case}, L={L}, T={T}, {rounds} rounds")
    y, st = _verify_run(cfg, work, T, dev)
    yref, Href = orc_mod.verify_rounds(work)
    assert_rows_close(y, yref, what=f"verify outputs ({case})")
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0
    if case == "C0":
        x = work.steps.x.reshape((rounds, T) + work.steps.x.shape[1:])
        want = work.D.astype(np.float32)[None, None, None, :, None] * x.astype(np.float32)
        assert np.array_equal(y, want), "C = 0: the draft outputs are not exactly D x"


# ---- status contract ---------------------------------------------------------------


def _two_states(cfg, work, dev, read_copy):
    p = staging.params(work, dev)
    sts = [staging.replay_state(cfg, work, dev) for _ in range(2)]
    if read_copy:
        for st in sts:
            rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
    return p, sts


@pytest.mark.parametrize("read_copy", [None, "e4m3"])
def test_one_head_copy_disagreeing_sets_status(read_copy):
    """Sequence 1's head 37 holds a ring pointer that is in range but differs
    from its other heads' copies (before and after the call).  A decode step
    sets RSSM_STATUS_META, writes NaN for head 37 of sequence 1 (and at most the
    other heads its workgroup serves), leaves that copy as it was, and every
    other output is bit-identical to a clean run."""
    dev = device()
    shape = synth.LayerShape(batch=3, window=4, max_drafts=2, **NEMO)
    work = synth.decode_workload(shape, 1, seed=1151, n0=1)
    cfg = staging.config(shape, read_copy=read_copy)
    p, (clean, dirty) = _two_states(cfg, work, dev, read_copy)
    dirty.meta[1, 37, 1] = 3                          # others hold {0, 1} now and {0, 2} after the call
    tok = staging.tokens_block(work.steps, 0, 1, dev)
    y = [torch.zeros((3, 1, cfg.nheads, cfg.headdim), device=dev) for _ in range(2)]
    say(f"one head's pointer copy disagrees (copy={read_copy})")
    rb.replayssm_decode_step(cfg, clean, p, tok, y[0])
    rb.replayssm_decode_step(cfg, dirty, p, tok, y[1])
    torch.cuda.synchronize()
    yc, yd = host(y[0]), host(y[1])
    assert host(clean.status)[0] == 0
    assert host(dirty.status)[0] & rb.RSSM_STATUS_META
    assert np.isnan(yd[1, 0, 37]).all()
    assert np.array_equal(yd[[0, 2]], yc[[0, 2]])
    nan_heads = [h for h in range(cfg.nheads) if np.isnan(yd[1, 0, h]).all()]
    assert set(nan_heads) <= set(range(36, 40)), nan_heads           # at most head 37's workgroup
    for h in set(range(cfg.nheads)) - set(nan_heads):
        assert np.array_equal(yd[1, 0, h], yc[1, 0, h]), h
    md, mc = host(dirty.meta), host(clean.meta)
    assert md[1, 37, 1] == 3
    assert np.array_equal(np.delete(md, nan_heads, axis=1)[1], np.delete(mc, nan_heads, axis=1)[1])
    # the commit kernel checks the copies the same way
    dirty.status.zero_()
    acc = torch.tensor([1, 1, 1], dtype=torch.int32, device=dev)
    rb.replayssm_commit(cfg, dirty, acc, 1)
    torch.cuda.synchronize()
    assert host(dirty.status)[0] & rb.RSSM_STATUS_META
    m2 = host(dirty.meta)
    assert m2[1, 37, 1] == 3
    assert np.all(m2[0, :, 1] == md[0, :, 1] + 1)


def test_first_head_copy_disagreeing_sets_status():
    """The reference copy itself (head 0's) disagrees with the others: the
    other heads of that sequence report it; other sequences bit-identical."""
    dev = device()
    shape = synth.LayerShape(batch=3, window=4, max_drafts=2, **NEMO)
    work = synth.decode_workload(shape, 1, seed=1152, n0=1)
    cfg = staging.config(shape)
    p, (clean, dirty) = _two_states(cfg, work, dev, None)
    dirty.meta[2, 0, 1] = 3
    tok = staging.tokens_block(work.steps, 0, 1, dev)
    y = [torch.zeros((3, 1, cfg.nheads, cfg.headdim), device=dev) for _ in range(2)]
    say("head 0's pointer copy disagrees")
    rb.replayssm_decode_step(cfg, clean, p, tok, y[0])
    rb.replayssm_decode_step(cfg, dirty, p, tok, y[1])
    torch.cuda.synchronize()
    yc, yd = host(y[0]), host(y[1])
    assert host(dirty.status)[0] & rb.RSSM_STATUS_META
    assert np.isnan(yd[2, 0, 1:]).all()
    assert np.array_equal(yd[:2], yc[:2])


def test_double_commit_overfilling_the_ring_sets_status():
    """Two commits without a verification in between leave sequence 1 with
    n = cap records; the next call would fold them and append its token past
    them, one slot beyond the ring: RSSM_STATUS_META, NaN outputs for that
    sequence, its pointer and checkpoint untouched, the other sequences
    bit-identical to a run whose second commit accepts nothing."""
    dev = device()
    L, T = 4, 3
    shape = synth.LayerShape(batch=3, window=L, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, 1, T, seed=1161, n0=np.array([1, 3, 2], np.int32))
    cfg = staging.config(shape)                           # cap = 9
    p, (clean, dirty) = _two_states(cfg, work, dev, None)
    drafts = staging.tokens_block(work.steps, 0, T, dev)
    yv = torch.empty((3, T, cfg.nheads, cfg.headdim), device=dev)
    first = torch.tensor([1, 3, 1], dtype=torch.int32, device=dev)
    later = synth.decode_workload(shape, 1, seed=1162)
    tok = staging.tokens_block(later.steps, 0, 1, dev)
    y = []
    for st, second in ((clean, [0, 0, 0]), (dirty, [0, 3, 0])):
        rb.replayssm_verify_drafts(cfg, st, p, drafts, yv)
        rb.replayssm_commit(cfg, st, first, T)
        rb.replayssm_commit(cfg, st, torch.tensor(second, dtype=torch.int32, device=dev), T)
        y.append(torch.zeros((3, 1, cfg.nheads, cfg.headdim), device=dev))
    torch.cuda.synchronize()
    assert host(dirty.meta)[1, 0, 1] == cfg.cap == 9
    ck_before = host(dirty.ckpt[1])
    say("decode after a double commit (n = cap)")
    rb.replayssm_decode_step(cfg, clean, p, tok, y[0])
    rb.replayssm_decode_step(cfg, dirty, p, tok, y[1])
    torch.cuda.synchronize()
    assert host(clean.status)[0] == 0
    assert host(dirty.status)[0] & rb.RSSM_STATUS_META
    yc, yd = host(y[0]), host(y[1])
    assert np.isnan(yd[1]).all()
    assert np.array_equal(yd[[0, 2]], yc[[0, 2]])
    assert np.all(host(dirty.meta)[1, :, 1] == cfg.cap)
    assert np.array_equal(host(dirty.ckpt[1]), ck_before)


def test_gdn_double_commit_overfilling_the_ring_sets_status():
    """The same double commit on the Gated DeltaNet layer: the call that would
    fold n = cap records and append past them is rejected for that sequence."""
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd import synth_gdn as sg
    from mamba_state_replay_amd.staging import GdnTokenStream
    dev = device()
    T = 3
    shape = sg.GdnShape(batch=3, nv=8, nk=4, dk=128, dv=128, window=4)
    w = sg.gdn_workload(shape, 2, 1171, "bf16", T=T)
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, T, "bf16")
    ts = GdnTokenStream(w.steps, dev, T)
    dec = GdnTokenStream(sg.gdn_workload(shape, 1, 1172, "bf16").steps, dev)
    o = []
    sts = []
    for second in ([0, 0, 0], [0, 3, 0]):
        st = bg.GdnState.allocate(cfg, dev)
        st.ckpt.copy_(torch.from_numpy(w.S0).to(dev))
        ov = torch.empty((shape.batch, T, shape.nv, shape.dv), device=dev)
        for r, acc in enumerate(([1, 3, 2], [1, 3, 1])):    # sequence 1: n = 6 after two rounds
            bg.gdn_verify_drafts(cfg, st, ts.call(r), ov)
            bg.gdn_commit(cfg, st, torch.tensor(acc, dtype=torch.int32, device=dev), T)
        bg.gdn_commit(cfg, st, torch.tensor(second, dtype=torch.int32, device=dev), T)
        sts.append(st)
    torch.cuda.synchronize()
    clean, dirty = sts
    assert int(dirty.meta.cpu().numpy()[1, 0, 0, 1]) == cfg.cap == 9
    ck_before = dirty.ckpt[1].cpu().clone()
    say("gdn decode after a double commit (n = cap)")
    for st in sts:
        o.append(torch.zeros((shape.batch, 1, shape.nv, shape.dv), device=dev))
        bg.gdn_decode_step(cfg, st, dec.call(0), o[-1])
    torch.cuda.synchronize()
    assert int(clean.status.cpu()[0]) == 0
    assert int(dirty.status.cpu()[0]) & 1
    oc, od = o[0].cpu().numpy(), o[1].cpu().numpy()
    assert np.isnan(od[1]).all()
    assert np.array_equal(od[[0, 2]], oc[[0, 2]])
    assert np.all(dirty.meta.cpu().numpy()[1, ..., 1] == cfg.cap)
    assert torch.equal(dirty.ckpt[1].cpu(), ck_before)


def test_gdn_one_copy_disagreeing_sets_status():
    """One workgroup's copy of a GDN sequence's ring pointer (value head 5,
    second row block) disagrees with the sequence's first copy: status bit,
    NaN for those 64 rows of head 5, everything else bit-identical."""
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd import synth_gdn as sg
    from mamba_state_replay_amd.staging import GdnTokenStream
    dev = device()
    shape = sg.GdnShape(batch=3, nv=8, nk=4, dk=128, dv=128, window=4)
    w = sg.gdn_workload(shape, 1, 1181, "bf16")
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, 1, "bf16")
    ts = GdnTokenStream(w.steps, dev)
    sts = []
    for _ in range(2):
        st = bg.GdnState.allocate(cfg, dev)
        st.ckpt.copy_(torch.from_numpy(w.S0).to(dev))
        sts.append(st)
    clean, dirty = sts
    parts = dirty.meta.shape[2]
    dirty.meta[1, 5, parts - 1, 1] = 2                    # others hold {0, 0} now and {0, 1} after the call
    o = [torch.zeros((shape.batch, 1, shape.nv, shape.dv), device=dev) for _ in range(2)]
    say("gdn one pointer copy disagrees")
    bg.gdn_decode_step(cfg, clean, ts.call(0), o[0])
    bg.gdn_decode_step(cfg, dirty, ts.call(0), o[1])
    torch.cuda.synchronize()
    assert int(dirty.status.cpu()[0]) & 1
    oc, od = o[0].cpu().numpy(), o[1].cpu().numpy()
    rows = shape.dv // parts
    bad = np.zeros(od.shape, bool)
    bad[1, 0, 5, (parts - 1) * rows:] = True
    assert np.isnan(od[bad]).all()
    assert np.array_equal(od[~bad], oc[~bad])
