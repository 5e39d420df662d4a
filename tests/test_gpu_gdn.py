"""GPU parity of the Gated DeltaNet entry points against the fp64 oracle
(oracle/gdn.py): decode with flushes, verify + commit rounds, the standalone
flush, the conventional kernel, pointer semantics and data-error handling."""
import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from mamba_state_replay_amd import synth_gdn as sg
from tests.gpu_util import TOL, assert_rows_close, head_err, say

pytestmark = pytest.mark.gpu

TINY = sg.GdnShape(batch=3, nv=4, nk=2, dk=16, dv=32, window=4)
LAYER_SMALL = sg.GdnShape(batch=3, nv=32, nk=16, dk=128, dv=128, window=16)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _bg():
    from mamba_state_replay_amd import binding_gdn as bg
    return bg


def _cfg(shape, T, in_dtype):
    bg = _bg()
    return bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, T, in_dtype)


def _state(cfg, S0, dev):
    st = _bg().GdnState.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(np.ascontiguousarray(S0)).to(dev))
    return st


def state_err(got, ref):
    """Per (sequence, head) state error normalized by the head's largest |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref).max(axis=(-1, -2)) / np.maximum(np.abs(ref).max(axis=(-1, -2)), 1e-30)


def _decode(shape, steps, seed, in_dtype, dev):
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    w = sg.gdn_workload(shape, steps, seed, in_dtype)
    cfg = _cfg(shape, 1, in_dtype)
    st = _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev)
    o = torch.empty((steps, shape.batch, 1, shape.nv, shape.dv), device=dev)
    say(f"gdn decode {shape} steps={steps} {in_dtype}")
    for t in range(steps):
        bg.gdn_decode_step(cfg, st, ts.call(t), o[t])
    torch.cuda.synchronize()
    return w, cfg, st, o.cpu().numpy()[:, :, 0]


@pytest.mark.parametrize("shape,steps,in_dtype", [(TINY, 23, "f32"), (TINY, 23, "bf16"),
                                                  (LAYER_SMALL, 37, "bf16"), (LAYER_SMALL, 21, "f32")],
                         ids=["tiny-f32", "tiny-bf16", "layer-bf16", "layer-f32"])
def test_gdn_decode_and_flush(shape, steps, in_dtype, dev):
    """Decode from an empty buffer through several flushes; outputs and, after
    a final flush, the checkpoint match stepping the gated delta rule."""
    bg = _bg()
    w, cfg, st, og = _decode(shape, steps, 31, in_dtype, dev)
    t = w.steps
    Sref, oref = ogdn.conventional(w.S0, t.q, t.k, t.v, t.g, t.beta)
    assert_rows_close(og, oref, what="gdn decode outputs")
    say("gdn flush")
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    err = state_err(st.ckpt.cpu().numpy(), Sref)
    print(f"[gpu] gdn flushed state: max error per head {err.max():.2e}", flush=True)
    assert err.max() <= TOL
    meta = st.meta.cpu().numpy()
    assert np.all(meta[..., 1] == 0) and np.all(meta == meta[:1, :1, :1])
    assert int(st.status.cpu()[0]) == 0


@pytest.mark.parametrize("shape,T,rounds,in_dtype", [(TINY, 3, 9, "f32"), (TINY, 2, 9, "bf16"),
                                                     (LAYER_SMALL, 3, 12, "bf16"),
                                                     (LAYER_SMALL, 1, 20, "bf16"),
                                                     (LAYER_SMALL, 4, 8, "f32")],
                         ids=["tiny-T3-f32", "tiny-T2-bf16", "layer-T3", "layer-T1", "layer-T4-f32"])
def test_gdn_verify_commit(shape, T, rounds, in_dtype, dev):
    """Speculative rounds: every draft's output equals stepping the accepted
    tokens so far and then the drafts; rollback is a pointer move, so the
    final checkpoint equals stepping only the accepted drafts."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    w = sg.gdn_workload(shape, rounds, 41 + T, in_dtype, T=T)
    acc = w.extra["accepted"]
    cfg = _cfg(shape, T, in_dtype)
    st = _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    say(f"gdn verify {shape} T={T} rounds={rounds} {in_dtype}")
    for r in range(rounds):
        bg.gdn_verify_drafts(cfg, st, ts.call(r), o[r])
        bg.gdn_commit(cfg, st, acc_d[r], T)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    tk = w.steps
    S = w.S0.astype(np.float64)
    oref = np.zeros((rounds, T, shape.batch, shape.nv, shape.dv))
    for r in range(rounds):
        sl = slice(r * T, (r + 1) * T)
        args = (tk.q[sl], tk.k[sl], tk.v[sl], tk.g[sl], tk.beta[sl])
        _, oref[r] = ogdn.conventional(S, *args)
        S, _ = ogdn.conventional(S, *args, nsteps=acc[r])
    og = np.swapaxes(o.cpu().numpy(), 1, 2)      # [rounds][T][batch][nv][dv]
    assert_rows_close(og, oref, what="gdn draft outputs")
    err = state_err(st.ckpt.cpu().numpy(), S)
    print(f"[gpu] gdn state after rounds: max error per head {err.max():.2e}", flush=True)
    assert err.max() <= TOL
    assert int(st.status.cpu()[0]) == 0


@pytest.mark.parametrize("shape,T,rounds,in_dtype", [(TINY, 3, 7, "f32"), (LAYER_SMALL, 3, 6, "bf16"),
                                                     (LAYER_SMALL, 2, 6, "bf16")],
                         ids=["tiny-T3", "layer-T3", "layer-T2"])
def test_gdn_snapshot_verify_baseline(shape, T, rounds, in_dtype, dev):
    """The conventional kernel with one snapshot per draft (nslots = T + 1) and
    its slot commit: draft outputs and the committed slot's state match the
    oracle stepping the accepted tokens."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    w = sg.gdn_workload(shape, rounds, 55 + T, in_dtype, T=T)
    acc = w.extra["accepted"]
    cfg = _cfg(shape, T, in_dtype)
    ns = T + 1
    states = torch.zeros((shape.batch, ns, shape.nv, shape.dv, shape.dk), device=dev)
    states[:, 0] = torch.from_numpy(w.S0).to(dev)
    slot = torch.zeros(shape.batch, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    say(f"gdn snapshot verify {shape} T={T}")
    for r in range(rounds):
        bg.gdn_conventional_update(cfg, states, ts.call(r), o[r], nslots=ns, slot=slot, status=status)
        bg.gdn_conventional_commit(cfg, slot, ns, acc_d[r], T, status)
    torch.cuda.synchronize()
    tk = w.steps
    S = w.S0.astype(np.float64)
    oref = np.zeros((rounds, T, shape.batch, shape.nv, shape.dv))
    for r in range(rounds):
        sl = slice(r * T, (r + 1) * T)
        args = (tk.q[sl], tk.k[sl], tk.v[sl], tk.g[sl], tk.beta[sl])
        _, oref[r] = ogdn.conventional(S, *args)
        S, _ = ogdn.conventional(S, *args, nsteps=acc[r])
    assert_rows_close(np.swapaxes(o.cpu().numpy(), 1, 2), oref, what="gdn snapshot-verify outputs")
    cur = slot.cpu().numpy()
    assert np.array_equal(cur, np.sum(acc, axis=0) % ns)
    got = states.cpu().numpy()[np.arange(shape.batch), cur]
    assert state_err(got, S).max() <= TOL
    assert int(status.cpu()[0]) == 0


@pytest.mark.parametrize("shape,in_dtype", [(TINY, "f32"), (LAYER_SMALL, "bf16")], ids=["tiny", "layer"])
def test_gdn_conventional_kernel(shape, in_dtype, dev):
    """The conventional GDN step (baseline) matches the oracle step by step."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    steps = 9
    w = sg.gdn_workload(shape, steps, 51, in_dtype)
    cfg = _cfg(shape, 1, in_dtype)
    S = torch.from_numpy(w.S0.copy()).to(dev)
    ts = GdnTokenStream(w.steps, dev)
    o = torch.empty((steps, shape.batch, 1, shape.nv, shape.dv), device=dev)
    say(f"gdn conventional {shape} {in_dtype}")
    for t in range(steps):
        bg.gdn_conventional_update(cfg, S, ts.call(t), o[t])
    torch.cuda.synchronize()
    tk = w.steps
    Sref, oref = ogdn.conventional(w.S0, tk.q, tk.k, tk.v, tk.g, tk.beta)
    assert_rows_close(o.cpu().numpy()[:, :, 0], oref, what="gdn conventional outputs")
    assert state_err(S.cpu().numpy(), Sref).max() <= TOL


def test_gdn_decode_equals_verify_one_and_commit(dev):
    """decode_step is verify(T=1) + commit(1), bit for bit, flushes included."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = LAYER_SMALL
    steps = 20
    w = sg.gdn_workload(shape, steps, 61)
    cfg = _cfg(shape, 1, "bf16")
    a, b = _state(cfg, w.S0, dev), _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev)
    one = torch.ones(shape.batch, dtype=torch.int32, device=dev)
    oa = torch.empty((steps, shape.batch, 1, shape.nv, shape.dv), device=dev)
    ob = torch.empty_like(oa)
    say("gdn decode vs verify(1)+commit(1)")
    for t in range(steps):
        bg.gdn_decode_step(cfg, a, ts.call(t), oa[t])
        bg.gdn_verify_drafts(cfg, b, ts.call(t), ob[t])
        bg.gdn_commit(cfg, b, one, 1)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert torch.equal(a.ckpt, b.ckpt) and torch.equal(a.meta, b.meta)


def test_gdn_records_beyond_pointer_are_never_read(dev):
    """Poison every ring slot outside the committed window with NaN before each
    call: outputs are unchanged (records past the pointer are ignored)."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = TINY
    T, rounds = 2, 10
    w = sg.gdn_workload(shape, rounds, 71, "f32", T=T)
    acc = torch.from_numpy(w.extra["accepted"]).to(dev)
    cfg = _cfg(shape, T, "f32")
    clean, dirty = _state(cfg, w.S0, dev), _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev, T)
    oc = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    od = torch.empty_like(oc)
    cap = cfg.cap
    say("gdn poisoned ring slots")
    for r in range(rounds):
        meta = dirty.meta.cpu().numpy()
        for bb in range(shape.batch):
            start, n = int(meta[bb, 0, 0, 0]), int(meta[bb, 0, 0, 1])
            live = {(start + c) % cap for c in range(n)}
            for s in range(cap):
                if s not in live:
                    dirty.buf_u[bb, :, s] = float("nan")
                    dirty.buf_g[bb, :, s] = float("nan")
                    dirty.buf_k[bb, :, s] = float("nan")
        bg.gdn_verify_drafts(cfg, clean, ts.call(r), oc[r])
        bg.gdn_verify_drafts(cfg, dirty, ts.call(r), od[r])
        bg.gdn_commit(cfg, clean, acc[r], T)
        bg.gdn_commit(cfg, dirty, acc[r], T)
        torch.cuda.synchronize()
    assert torch.isfinite(od).all()
    assert torch.equal(oc, od)


def test_gdn_bad_pointer_sets_status(dev):
    """A ring pointer out of range: status bit, NaN outputs for that sequence,
    its state untouched; the other sequences proceed."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = TINY
    w = sg.gdn_workload(shape, 1, 81, "f32")
    cfg = _cfg(shape, 1, "f32")
    st = _state(cfg, w.S0, dev)
    st.meta[1, :, :, 0] = cfg.cap + 3
    ts = GdnTokenStream(w.steps, dev)
    o = torch.zeros((shape.batch, 1, shape.nv, shape.dv), device=dev)
    say("gdn corrupt ring pointer (rejected by the kernel's own check)")
    bg.gdn_decode_step(cfg, st, ts.call(0), o)
    torch.cuda.synchronize()
    assert int(st.status.cpu()[0]) & 1
    on = o.cpu().numpy()
    assert np.all(np.isnan(on[1])) and np.all(np.isfinite(on[[0, 2]]))
    assert torch.equal(st.ckpt[1].cpu(), torch.from_numpy(w.S0[1]))
    assert np.all(st.meta[1].cpu().numpy()[..., 0] == cfg.cap + 3)


def test_gdn_commit_rejects_bad_counts(dev):
    bg = _bg()
    cfg = _cfg(TINY, 2, "f32")
    st = bg.GdnState.allocate(cfg, dev)
    acc = torch.tensor([0, 3, 1], dtype=torch.int32, device=dev)
    say("gdn commit with an accepted count above T")
    bg.gdn_commit(cfg, st, acc, 2)
    torch.cuda.synchronize()
    assert int(st.status.cpu()[0]) & 2
    m = st.meta.cpu().numpy()
    assert np.all(m[0, ..., 1] == 0) and np.all(m[1, ..., 1] == 0) and np.all(m[2, ..., 1] == 1)


FULL = sg.GdnShape(batch=512, nv=32, nk=16, dk=128, dv=128, window=16)
SAMPLE = [0, 137, 300, 511]


def test_gdn_fullsize_decode_sampled(dev):
    """The benchmarked GDN launch (batch 512, 32 value heads, dk = dv = 128,
    L = 16, bf16 inputs, seed of the bench): 20 decode steps (one flush) over
    the whole batch, then a flush; sampled sequences against the oracle."""
    bg = _bg()
    steps = 20
    w, cfg, st, og = _decode(FULL, steps, 2001, "bf16", dev)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    t = w.steps
    sl = np.array(SAMPLE)
    Sref, oref = ogdn.conventional(w.S0[sl], t.q[:, sl], t.k[:, sl], t.v[:, sl], t.g[:, sl], t.beta[:, sl])
    assert_rows_close(og[:, sl], oref, what="gdn full-size decode outputs (sampled)")
    err = state_err(st.ckpt[torch.from_numpy(sl).to(dev)].cpu().numpy(), Sref)
    assert err.max() <= TOL
    assert int(st.status.cpu()[0]) == 0


def test_gdn_fullsize_verify_sampled(dev):
    """Speculative rounds at the benchmarked size (batch 512, T = 3, U{0..3}
    acceptance): sampled sequences' draft outputs and final state."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    T, rounds = 3, 8
    w = sg.gdn_workload(FULL, rounds, 2003, "bf16", T=T)
    acc = w.extra["accepted"]
    cfg = _cfg(FULL, T, "bf16")
    st = _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, FULL.batch, T, FULL.nv, FULL.dv), device=dev)
    say(f"gdn full-size verify T={T} rounds={rounds}")
    for r in range(rounds):
        bg.gdn_verify_drafts(cfg, st, ts.call(r), o[r])
        bg.gdn_commit(cfg, st, acc_d[r], T)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    sl = np.array(SAMPLE)
    tk = w.steps
    S = w.S0[sl].astype(np.float64)
    oref = np.zeros((rounds, T, len(sl), FULL.nv, FULL.dv))
    for r in range(rounds):
        rs = slice(r * T, (r + 1) * T)
        args = (tk.q[rs][:, sl], tk.k[rs][:, sl], tk.v[rs][:, sl], tk.g[rs][:, sl], tk.beta[rs][:, sl])
        _, oref[r] = ogdn.conventional(S, *args)
        S, _ = ogdn.conventional(S, *args, nsteps=acc[r][sl])
    og = np.swapaxes(o.cpu().numpy()[:, sl], 1, 2)
    assert_rows_close(og, oref, what="gdn full-size draft outputs (sampled)")
    assert state_err(st.ckpt[torch.from_numpy(sl).to(dev)].cpu().numpy(), S).max() <= TOL
    assert int(st.status.cpu()[0]) == 0


def _clone_gdn(st):
    bg = _bg()
    return bg.GdnState(**{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in vars(st).items()})


@pytest.mark.parametrize("ckpt", ["f32", "f16"])
def test_gdn_graph_replays_match_eager(ckpt, dev):
    """GDN decode steps (flushes included) and verify + commit rounds captured
    in one HIP graph: three replays, each after eager launches of the same
    tokens on a twin state and a synchronisation, reproduce the eager results
    bit for bit (the entry points only launch kernels on the caller's stream)."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = sg.GdnShape(batch=4, nv=32, nk=16, dk=128, dv=128, window=4)
    K, T, R = 9, 3, 3
    w = sg.gdn_workload(shape, K, 91)
    vw = sg.gdn_workload(shape, R, 92, T=T)
    cfg1, cfgT = (bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, t, "bf16", ckpt)
                  for t in (1, T))
    ts, vts = GdnTokenStream(w.steps, dev), GdnTokenStream(vw.steps, dev, T)
    acc = torch.from_numpy(vw.extra["accepted"]).to(dev)
    d_e, d_g = _state(cfg1, w.S0, dev), None
    d_g = _clone_gdn(d_e)
    v_e = _state(cfgT, vw.S0, dev)
    v_g = _clone_gdn(v_e)
    o_e = torch.empty((K, shape.batch, 1, shape.nv, shape.dv), device=dev)
    o_g = torch.empty_like(o_e)
    vo_e = torch.empty((R, shape.batch, T, shape.nv, shape.dv), device=dev)
    vo_g = torch.empty_like(vo_e)

    def run(dstate, vstate, o, vo):
        for t in range(K):
            bg.gdn_decode_step(cfg1, dstate, ts.call(t), o[t])
        for r in range(R):
            bg.gdn_verify_drafts(cfgT, vstate, vts.call(r), vo[r])
            bg.gdn_commit(cfgT, vstate, acc[r], T)

    say(f"capture GDN decode and verify + commit ({ckpt} checkpoint)")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(d_g, v_g, o_g, vo_g)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"GDN eager pass {rep}")
        run(d_e, v_e, o_e, vo_e)
        torch.cuda.synchronize()
        say(f"GDN graph replay {rep}")
        o_g.fill_(float("nan"))
        vo_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(vo_g, vo_e), f"replay {rep} differs"
        for a, b in ((d_g, d_e), (v_g, v_e)):
            assert torch.equal(a.ckpt, b.ckpt) and torch.equal(a.meta, b.meta)
            assert torch.equal(a.buf_u, b.buf_u) and torch.equal(a.buf_k, b.buf_k)
    assert int(d_g.status.cpu()[0]) == 0 and int(v_g.status.cpu()[0]) == 0


def test_gdn_long_run_no_drift(dev):
    """160 decode steps at L = 16 (ten flushes) on the layer shape: the error
    against the fp64 oracle stays at the fp32 level in every window, with no
    growth from the first windows to the last."""
    shape = sg.GdnShape(batch=2, nv=32, nk=16, dk=128, dv=128, window=16)
    steps = 160
    w, cfg, st, og = _decode(shape, steps, 97, "bf16", dev)
    t = w.steps
    _, oref = ogdn.conventional(w.S0, t.q, t.k, t.v, t.g, t.beta)
    errs = []
    for k in range(steps // 16):
        sl = slice(16 * k, 16 * (k + 1))
        errs.append(float(head_err(og[sl], oref[sl]).max()))
    print(f"[gpu] gdn per-window max error: first {errs[:3]}, last {errs[-3:]}", flush=True)
    assert max(errs) <= TOL
    assert max(errs[-3:]) <= 4 * max(max(errs[:3]), 1e-7)


@pytest.mark.parametrize("shape,T,rounds", [
    (sg.GdnShape(batch=2, nv=4, nk=2, dk=16, dv=32, window=64), 8, 14),        # RSSM_MAX_WINDOW, RSSM_MAX_DRAFTS
    (sg.GdnShape(batch=2, nv=32, nk=16, dk=128, dv=128, window=40), 8, 9),     # largest window at T = 8 in 64 KiB LDS
    (sg.GdnShape(batch=1, nv=32, nk=16, dk=128, dv=128, window=64), 4, 20),    # largest window at T = 4
], ids=["tiny-L64-T8", "layer-L40-T8", "layer-L64-T4-batch1"])
def test_gdn_window_and_draft_limits(shape, T, rounds, dev):
    """Verify + commit at the largest windows and draft counts the library
    accepts: outputs and the flushed state match the oracle."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    w = sg.gdn_workload(shape, rounds, 131 + T, "bf16", T=T)
    acc = w.extra["accepted"]
    cfg = _cfg(shape, T, "bf16")
    st = _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    say(f"gdn limits {shape} T={T} rounds={rounds}")
    for r in range(rounds):
        bg.gdn_verify_drafts(cfg, st, ts.call(r), o[r])
        bg.gdn_commit(cfg, st, acc_d[r], T)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    tk = w.steps
    S = w.S0.astype(np.float64)
    oref = np.zeros((rounds, T, shape.batch, shape.nv, shape.dv))
    for r in range(rounds):
        sl = slice(r * T, (r + 1) * T)
        args = (tk.q[sl], tk.k[sl], tk.v[sl], tk.g[sl], tk.beta[sl])
        _, oref[r] = ogdn.conventional(S, *args)
        S, _ = ogdn.conventional(S, *args, nsteps=acc[r])
    assert_rows_close(np.swapaxes(o.cpu().numpy(), 1, 2), oref, what="gdn outputs at the limits")
    assert state_err(st.ckpt.cpu().numpy(), S).max() <= TOL
    assert int(st.status.cpu()[0]) == 0


@pytest.mark.parametrize("ckpt", ["f32", "f16"])
def test_gdn_commit_verify_equals_commit_then_verify(ckpt, dev):
    """The fused entry point (commit of round r-1 inside verify of round r) gives
    bit-identical outputs, checkpoints and rings to commit + verify; an accepted
    count above T_prev is flagged and that sequence's outputs are NaN."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = sg.GdnShape(batch=3, nv=32, nk=16, dk=128, dv=128, window=4)
    T, rounds = 3, 7
    w = sg.gdn_workload(shape, rounds, 151, "bf16", T=T)
    cfg = bg.GdnConfig(shape.batch, shape.nv, shape.nk, shape.dk, shape.dv, shape.window, T, "bf16", ckpt)
    S0 = torch.from_numpy(w.S0).to(dev).to(cfg.ckpt_torch)
    a, f = bg.GdnState.allocate(cfg, dev), bg.GdnState.allocate(cfg, dev)
    a.ckpt.copy_(S0)
    f.ckpt.copy_(S0)
    ts = GdnTokenStream(w.steps, dev, T)
    acc = torch.from_numpy(w.extra["accepted"]).to(dev)
    oa = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    of = torch.empty_like(oa)
    say(f"gdn commit+verify fused vs separate ({ckpt})")
    for r in range(rounds):
        tok = ts.call(r)
        tok.sr_seed = 40 + r
        if r == 0:
            bg.gdn_verify_drafts(cfg, f, tok, of[r])
        else:
            bg.gdn_commit_verify(cfg, f, acc[r - 1], T, tok, of[r])
        bg.gdn_verify_drafts(cfg, a, tok, oa[r])
        bg.gdn_commit(cfg, a, acc[r], T)
    bg.gdn_commit(cfg, f, acc[rounds - 1], T)
    torch.cuda.synchronize()
    assert torch.equal(oa, of)
    for x, y in ((a.ckpt, f.ckpt), (a.meta, f.meta), (a.buf_u, f.buf_u), (a.buf_k, f.buf_k), (a.buf_g, f.buf_g)):
        assert torch.equal(x, y)
    assert int(a.status.cpu()[0]) == 0 and int(f.status.cpu()[0]) == 0
    bad = torch.tensor([1, T + 1, 0], dtype=torch.int32, device=dev)
    o1 = torch.zeros((shape.batch, T, shape.nv, shape.dv), device=dev)
    meta_before = f.meta.clone()
    say("gdn commit+verify with an accepted count above T_prev")
    bg.gdn_commit_verify(cfg, f, bad, T, ts.call(0), o1)
    torch.cuda.synchronize()
    assert int(f.status.cpu()[0]) & 2
    assert torch.isnan(o1[1]).all() and torch.isfinite(o1[[0, 2]]).all()
    assert torch.equal(f.meta[1], meta_before[1])


@pytest.mark.parametrize("policy", ["all", "none", "alternate"])
def test_gdn_acceptance_extremes(policy, dev):
    """Every draft accepted each round (the ring at its fullest: L - 1 + T
    committed records before a flush), none ever accepted (the drafts' slots
    rewritten every round, the checkpoint never moves), and alternating T / 0:
    outputs and final state against the oracle."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = sg.GdnShape(batch=2, nv=32, nk=16, dk=128, dv=128, window=5)
    T, rounds = 3, 10
    w = sg.gdn_workload(shape, rounds, 171, "bf16", T=T)
    acc = {"all": np.full((rounds, shape.batch), T), "none": np.zeros((rounds, shape.batch)),
           "alternate": np.array([[T if (r + b) % 2 == 0 else 0 for b in range(shape.batch)]
                                  for r in range(rounds)])}[policy].astype(np.int32)
    cfg = _cfg(shape, T, "bf16")
    st = _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    say(f"gdn acceptance policy {policy}")
    for r in range(rounds):
        bg.gdn_verify_drafts(cfg, st, ts.call(r), o[r])
        bg.gdn_commit(cfg, st, acc_d[r], T)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    tk = w.steps
    S = w.S0.astype(np.float64)
    oref = np.zeros((rounds, T, shape.batch, shape.nv, shape.dv))
    for r in range(rounds):
        sl = slice(r * T, (r + 1) * T)
        args = (tk.q[sl], tk.k[sl], tk.v[sl], tk.g[sl], tk.beta[sl])
        _, oref[r] = ogdn.conventional(S, *args)
        S, _ = ogdn.conventional(S, *args, nsteps=acc[r])
    assert_rows_close(np.swapaxes(o.cpu().numpy(), 1, 2), oref, what=f"gdn outputs ({policy})")
    assert state_err(st.ckpt.cpu().numpy(), S).max() <= TOL
    if policy == "none":
        assert np.array_equal(st.ckpt.cpu().numpy(), w.S0)        # nothing committed: checkpoint untouched
    assert int(st.status.cpu()[0]) == 0


@pytest.mark.parametrize("nv,nk", [(8, 1), (4, 4), (16, 2)], ids=["8-per-key", "1-per-key", "8-per-key-2"])
def test_gdn_head_grouping(nv, nk, dev):
    """Value heads per key head from 1 to 8 (the key ring is appended by the
    first row block of each key head's first value head and read by all of
    them): verify + commit rounds and the flushed state against the oracle."""
    from mamba_state_replay_amd.staging import GdnTokenStream
    bg = _bg()
    shape = sg.GdnShape(batch=2, nv=nv, nk=nk, dk=128, dv=128, window=4)
    T, rounds = 2, 8
    w = sg.gdn_workload(shape, rounds, 191 + nv + nk, "bf16", T=T)
    acc = w.extra["accepted"]
    cfg = _cfg(shape, T, "bf16")
    st = _state(cfg, w.S0, dev)
    ts = GdnTokenStream(w.steps, dev, T)
    acc_d = torch.from_numpy(acc).to(dev)
    o = torch.empty((rounds, shape.batch, T, shape.nv, shape.dv), device=dev)
    say(f"gdn head grouping nv={nv} nk={nk}")
    for r in range(rounds):
        bg.gdn_verify_drafts(cfg, st, ts.call(r), o[r])
        bg.gdn_commit(cfg, st, acc_d[r], T)
    bg.gdn_flush(cfg, st)
    torch.cuda.synchronize()
    tk = w.steps
    S = w.S0.astype(np.float64)
    oref = np.zeros((rounds, T, shape.batch, shape.nv, shape.dv))
    for r in range(rounds):
        sl = slice(r * T, (r + 1) * T)
        args = (tk.q[sl], tk.k[sl], tk.v[sl], tk.g[sl], tk.beta[sl])
        _, oref[r] = ogdn.conventional(S, *args)
        S, _ = ogdn.conventional(S, *args, nsteps=acc[r])
    assert_rows_close(np.swapaxes(o.cpu().numpy(), 1, 2), oref, what=f"gdn outputs nv={nv} nk={nk}")
    assert state_err(st.ckpt.cpu().numpy(), S).max() <= TOL
    assert int(st.status.cpu()[0]) == 0
