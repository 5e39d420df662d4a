"""GDN layer with an FP16 recurrence checkpoint written with stochastic
rounding (ckpt_dtype "f16"): the flush writes the oracle's stochastic rounding
(oracle/sr.py, from the generator's and the rounding's definitions) of the
exact fold, and decoding through several flushes tracks the oracle that rounds
its own exact folds with the same seeds."""
import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from oracle import sr
from mamba_state_replay_amd import synth_gdn as sg
from tests.gpu_util import assert_rows_close, say

pytestmark = pytest.mark.gpu

SHAPE = sg.GdnShape(batch=2, nv=32, nk=16, dk=128, dv=128, window=4)
# dv = 128 runs the kernel with 128 rows per workgroup; dv = 64 and dk = 16 the 64- and 16-row one
SHAPES = {"wide": SHAPE, "rows64": sg.GdnShape(batch=2, nv=8, nk=4, dk=128, dv=64, window=4),
          "tiny": sg.GdnShape(batch=3, nv=4, nk=2, dk=16, dv=32, window=4)}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _setup(steps, seed, dev, T=1, shape=SHAPE):
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd.staging import GdnTokenStream
    w = sg.gdn_workload(shape, steps, seed)
    S0h = w.S0.astype(np.float16)                 # the checkpoint holds fp16 values
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, T, "bf16", "f16")
    st = bg.GdnState.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(S0h).to(dev))
    return bg, w, S0h.astype(np.float64), cfg, st, GdnTokenStream(w.steps, dev)


def _neighbours(got, exact, spacings=1):
    """|got - exact| minus `spacings` fp16 spacings at the element (the larger
    spacing at a binade edge) and 1e-6 of the head's largest magnitude for the
    fp32 fold's own rounding: <= 0 where got is that close to exact."""
    g64 = got.astype(np.float64)
    spacing = np.maximum(sr.f16_grid(np.abs(exact))[1], sr.f16_grid(np.abs(g64))[1])
    slack = 1e-6 * np.abs(exact).max(axis=(-1, -2), keepdims=True)
    return np.abs(g64 - exact) - spacings * spacing - slack


def _spacing_rows(ck):
    """2 ||spacing16(|ck[b, h, i, :]|)||_2 per state row [batch][nv][dv]: the
    largest l2 norm of a row difference whose elements are each at most one fp16
    spacing of the larger value's binade (at most twice the spacing at |ck|)."""
    _, sp = sr.f16_grid(np.abs(np.asarray(ck, np.float64)))
    return 2.0 * np.sqrt((sp ** 2).sum(axis=-1))


@pytest.mark.parametrize("which", sorted(SHAPES))
def test_gdn_f16_flush_writes_stochastic_rounding_of_the_fold(which, dev):
    shape = SHAPES[which]
    bg, w, S0, cfg, st, ts = _setup(4, 3001, dev, shape=shape)
    o = torch.empty((4, shape.batch, 1, shape.nv, shape.dv), device=dev)
    say(f"gdn f16 checkpoint ({which}): 4 decode steps, then a flush")
    for t in range(4):
        bg.gdn_decode_step(cfg, st, ts.call(t), o[t])
    seed = 0x5EED0000D17A
    bg.gdn_flush(cfg, st, seed)
    torch.cuda.synchronize()
    tk = w.steps
    exact, oref = ogdn.conventional(S0, tk.q, tk.k, tk.v, tk.g, tk.beta)
    assert_rows_close(o.cpu().numpy()[:, :, 0], oref, what="gdn f16 outputs before the flush")
    got = st.ckpt.cpu().numpy()
    want = sr.sr_checkpoint(exact, seed)
    same = got.view(np.uint16) == want.astype(np.float16).view(np.uint16)
    excess = _neighbours(got, exact)
    print(f"[gpu] gdn f16 flush: {same.mean():.6f} of elements equal the oracle's rounding; "
          f"largest excess over one spacing {excess.max():.3g}", flush=True)
    assert (excess <= 0).all(), "an element left the fp16 neighbours of its fold"
    assert same.mean() >= 0.999
    assert np.all(st.meta.cpu().numpy()[..., 1] == 0)


@pytest.mark.parametrize("which", sorted(SHAPES))
def test_gdn_f16_decode_through_flushes(which, dev):
    """Decode 13 tokens at L = 4 (flushes at the starts of calls 4, 8 and 12,
    each with its own seed).  The oracle composes the definition's stepping with
    the same flush schedule: at a flush it folds exactly (fp64), the flushing
    call's token reads the exact fold, and the checkpoint then becomes the
    stochastic rounding of that fold with the call's seed.  Outputs: the FP32
    tolerance per row plus what rounding decisions that went the other way can
    move them (bounded below)."""
    steps = 13
    SHAPE = SHAPES[which]
    bg, w, S0, cfg, st, ts = _setup(steps, 3002, dev, shape=SHAPE)
    o = torch.empty((steps, SHAPE.batch, 1, SHAPE.nv, SHAPE.dv), device=dev)
    say(f"gdn f16 checkpoint ({which}): 13 decode steps through three flushes")
    for t in range(steps):
        tok = ts.call(t)
        tok.sr_seed = 9000 + t
        bg.gdn_decode_step(cfg, st, tok, o[t])
    torch.cuda.synchronize()
    tk = w.steps
    rep = ogdn.Replay(S0, SHAPE.nv, SHAPE.nk)
    oref = np.zeros((steps, SHAPE.batch, SHAPE.nv, SHAPE.dv))
    # Where a rounding decision went the other way, the kernel's checkpoint row
    # differs from the oracle's by delta, at most one spacing per element.  The
    # gated delta rule carries it linearly: delta S_t = delta S_s M_t with M_t a
    # product of alpha (I - beta k k^T), whose l2 norm is at most 1 (unit keys,
    # 0 <= beta <= 1, alpha <= 1), and the next flush rounds F(S + delta) and
    # F(S) with the same random bits, which adds at most one spacing per element.
    # So after each flush a row's difference grows by at most _spacing_rows of
    # that flush's checkpoint, and an output row moves by at most that sum times
    # ||q_t||_2 (allowance below, on top of the FP32 tolerance per row).
    grow = np.zeros((SHAPE.batch, SHAPE.nv, SHAPE.dv))
    allow = np.zeros(oref.shape)
    hpk = SHAPE.nv // SHAPE.nk
    for t in range(steps):
        flushing = [b for b in range(SHAPE.batch) if len(rep.records[b]) >= SHAPE.window]
        for b in flushing:
            rep.fold(b)
        for b in range(SHAPE.batch):
            oref[t, b] = rep.step(b, tk.q[t][b], tk.k[t][b], tk.v[t][b], tk.g[t][b], tk.beta[t][b])
        qn = np.repeat(np.linalg.norm(np.asarray(tk.q[t], np.float64), axis=-1), hpk, axis=1)   # [batch][nv]
        allow[t] = grow * qn[:, :, None]
        if flushing:
            rounded = sr.sr_checkpoint(rep.ckpt, 9000 + t)
            rows = _spacing_rows(rounded)
            for b in flushing:
                rep.ckpt[b] = rounded[b]
                grow[b] += rows[b]
    assert_rows_close(o.cpu().numpy()[:, :, 0], oref, what="gdn f16 decode outputs", allowance=allow)
    # the checkpoint after the last flush (call 12) equals the oracle's almost
    # everywhere.  Where a rounding decision went the other way (the kernel's
    # fp32 fold and the oracle's fp64 fold straddle a threshold) the two differ
    # by a spacing, and in GDN such a difference spreads along its row at the
    # next tokens (u reads S k), so after three flushes the bound is on the
    # head's scale: within four fp16 half-ulps (2^-11) of the head's largest value
    got = st.ckpt.cpu().numpy()
    diff = np.abs(got.astype(np.float64) - rep.ckpt).max(axis=(-1, -2))
    scale = np.abs(rep.ckpt).max(axis=(-1, -2))
    print(f"[gpu] gdn f16 checkpoint after three flushes: max difference per head "
          f"{(diff / scale).max():.2e} of the head's largest value", flush=True)
    assert (diff <= 4 * 2.0 ** -11 * scale).all()
    same = got.view(np.uint16) == rep.ckpt.astype(np.float16).view(np.uint16)
    print(f"[gpu] gdn f16 checkpoint after three flushes: {same.mean():.6f} equal", flush=True)
    assert same.mean() >= 0.99
    assert int(st.status.cpu()[0]) == 0


@pytest.mark.parametrize("which", sorted(SHAPES))
def test_gdn_f16_verify_commit(which, dev):
    """Speculative rounds over the FP16 checkpoint (T = 3, L = 4): outputs match
    the oracle that follows the same flush schedule and rounding, within the
    FP32 tolerance per row plus the allowance of the decode test above for
    rounding decisions that went the other way (the drafts of a round read the
    exact fold of its flush; the rounded checkpoint serves the later rounds)."""
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd.staging import GdnTokenStream
    shape = SHAPES[which]
    T, rounds = 3, 6
    w = sg.gdn_workload(shape, rounds, 3003, T=T)
    acc = w.extra["accepted"]
    S0 = w.S0.astype(np.float16)
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, T, "bf16", "f16")
    st = bg.GdnState.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(S0).to(dev))
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    say(f"gdn f16 checkpoint ({which}): verify + commit rounds")
    for r in range(rounds):
        tok = ts.call(r)
        tok.sr_seed = 7000 + r
        bg.gdn_verify_drafts(cfg, st, tok, o[r])
        bg.gdn_commit(cfg, st, acc_d[r], T)
    torch.cuda.synchronize()
    tk = w.steps
    rep = ogdn.Replay(S0.astype(np.float64), shape.nv, shape.nk)
    oref = np.zeros((rounds, T, shape.batch, shape.nv, shape.dv))
    grow = np.zeros((shape.batch, shape.nv, shape.dv))
    allow = np.zeros(oref.shape)
    hpk = shape.nv // shape.nk
    for r in range(rounds):
        flushing = [b for b in range(shape.batch) if len(rep.records[b]) >= shape.window]
        for b in flushing:
            rep.fold(b)
        for b in range(shape.batch):
            drafts = [(tk.q[r * T + i][b], tk.k[r * T + i][b], tk.v[r * T + i][b], tk.g[r * T + i][b],
                       tk.beta[r * T + i][b]) for i in range(T)]
            outs, recs = rep.verify(b, drafts)
            oref[r, :, b] = np.stack(outs)
            rep.commit(b, recs, int(acc[r, b]))
        for i in range(T):
            qn = np.repeat(np.linalg.norm(np.asarray(tk.q[r * T + i], np.float64), axis=-1), hpk, axis=1)
            allow[r, i] = grow * qn[:, :, None]
        if flushing:
            rounded = sr.sr_checkpoint(rep.ckpt, 7000 + r)
            rows = _spacing_rows(rounded)
            for b in flushing:
                rep.ckpt[b] = rounded[b]
                grow[b] += rows[b]
    assert_rows_close(np.swapaxes(o.cpu().numpy(), 1, 2), oref, what=f"gdn f16 draft outputs ({which})",
                      allowance=allow)
    assert int(st.status.cpu()[0]) == 0


def test_gdn_f16_tracks_fp32_over_2048_steps(dev):
    """2048 decode steps at L = 16 with the FP16 checkpoint (128 flushes, each
    with its own rounding seed) beside the FP32 checkpoint, both against the
    exact fp64 recurrence from the same fp16-valued start (the replay form in
    fp64, pinned to the definition by the oracle tests).  The FP16 error sits
    at the fp16 level and does not grow from the first windows to the last."""
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd.staging import GdnTokenStream
    from tests.gpu_util import head_err
    shape = sg.GdnShape(batch=2, nv=8, nk=4, dk=128, dv=128, window=16)
    steps = 2048
    w = sg.gdn_workload(shape, steps, 3050)
    S0h = w.S0.astype(np.float16)
    ts = GdnTokenStream(w.steps, dev)
    outs = {}
    for ck in ("f32", "f16"):
        cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, 1, "bf16", ck)
        st = bg.GdnState.allocate(cfg, dev)
        st.ckpt.copy_(torch.from_numpy(S0h).to(dev).to(cfg.ckpt_torch))
        o = torch.empty((steps, shape.batch, 1, shape.nv, shape.dv), device=dev)
        say(f"gdn {ck} checkpoint: {steps} decode steps")
        for t in range(steps):
            tok = ts.call(t)
            tok.sr_seed = 123456 + t
            bg.gdn_decode_step(cfg, st, tok, o[t])
        torch.cuda.synchronize()
        assert int(st.status.cpu()[0]) == 0
        outs[ck] = o.cpu().numpy()[:, :, 0]
    tk = w.steps
    _, oref = ogdn.replay_decode(S0h.astype(np.float64), tk.q, tk.k, tk.v, tk.g, tk.beta, shape.window)
    win = 128
    errs = {ck: np.array([head_err(outs[ck][i:i + win], oref[i:i + win]).max() for i in range(0, steps, win)])
            for ck in outs}
    q = len(errs["f16"]) // 4
    print(f"[gpu] gdn 2048 steps, max error per window: fp32 {errs['f32'].max():.2e}; fp16 first quarter "
          f"{errs['f16'][:q].max():.2e}, last quarter {errs['f16'][-q:].max():.2e}", flush=True)
    assert errs["f32"].max() <= 1e-4
    assert errs["f16"].max() <= 2e-3                       # fp16 state: a few 2^-11 half-ulps
    assert errs["f16"][-q:].max() <= 2 * errs["f16"][:q].max()


def test_gdn_f16_fullsize_decode_sampled(dev):
    """The benchmarked FP16-checkpoint launch (batch 512, 32 value heads over
    16 key heads, dk = dv = 128, L = 16; the 128-row kernel): 17 decode steps,
    the flush at the start of call 16 with that call's seed.  Sampled sequences'
    outputs against the oracle, and their checkpoint after the flush against
    the stochastic rounding of the exact fold, taken at the elements' flat
    indices in the whole checkpoint (the generator's counters)."""
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd.staging import GdnTokenStream
    shape = sg.GdnShape(batch=512, nv=32, nk=16, dk=128, dv=128, window=16)
    steps, fseed = 17, 0xF16F0000 + 16
    sample = np.array([0, 137, 300, 511])
    w = sg.gdn_workload(shape, steps, 2001)
    S0h = w.S0.astype(np.float16)
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, 1, "bf16", "f16")
    st = bg.GdnState.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(S0h).to(dev))
    ts = GdnTokenStream(w.steps, dev)
    o = torch.empty((steps, shape.batch, 1, shape.nv, shape.dv), device=dev)
    say("gdn f16 checkpoint, batch 512: 17 decode steps, one flush")
    for t in range(steps):
        tok = ts.call(t)
        tok.sr_seed = fseed if t == 16 else 1 + t
        bg.gdn_decode_step(cfg, st, tok, o[t])
    torch.cuda.synchronize()
    tk = w.steps
    S0 = S0h[sample].astype(np.float64)
    args = [a[:, sample] for a in (tk.q, tk.k, tk.v, tk.g, tk.beta)]
    exact, oref = ogdn.conventional(S0, *[a[:16] for a in args])
    _, o16 = ogdn.conventional(exact, *[a[16:] for a in args])      # call 16 reads the exact fold
    oref = np.concatenate([oref, o16])
    assert_rows_close(o.cpu().numpy()[:, sample, 0], oref, what="gdn f16 batch-512 outputs (sampled)")
    per_seq = shape.nv * shape.dv * shape.dk
    idx = (sample.astype(np.uint64)[:, None] * np.uint64(per_seq)
           + np.arange(per_seq, dtype=np.uint64)[None, :]).reshape(exact.shape)
    want = sr.f16_sr(exact.astype(np.float32), sr.words(idx, fseed))
    got = st.ckpt[torch.from_numpy(sample).to(dev)].cpu().numpy()
    same = got.view(np.uint16) == want.astype(np.float16).view(np.uint16)
    excess = _neighbours(got, exact)
    print(f"[gpu] gdn f16 batch-512 flush: {same.mean():.6f} of sampled elements equal the oracle's "
          f"rounding; largest excess over one spacing {excess.max():.3g}", flush=True)
    assert (excess <= 0).all()
    assert same.mean() >= 0.999
    assert np.all(st.meta.cpu().numpy()[..., 1] == 1)
    assert int(st.status.cpu()[0]) == 0
