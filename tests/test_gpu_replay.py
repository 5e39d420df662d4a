"""GPU parity of the ReplaySSM decode / flush / verify / commit kernels vs the fp64 oracle.

The oracle steps the conventional recurrence token by token in fp64; the HIP
path keeps a checkpoint plus records and must agree within max relative
error 1e-4 per (sequence, head, token) row.
"""
import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from tests.gpu_util import assert_rows_close, device, host, say, tile_err, TOL

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)


def run_decode(cfg, work, nsteps, dev, state=None):
    st = state or staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps.slice(0, nsteps), dev)
    y = torch.empty((nsteps, cfg.batch, 1, cfg.nheads, cfg.headdim), dtype=torch.float32, device=dev)
    for t in range(nsteps):
        rb.replayssm_decode_step(cfg, st, p, stream.call(t), y[t])
    torch.cuda.synchronize()
    return host(y)[:, :, 0], st, p


def test_decode_tiny_f32():
    """Tiny layer: batch 1, 4 heads, 16x16 tiles, L=4, 64 steps, h0 = 0, fp32 inputs."""
    dev = device()
    shape = synth.TINY
    work = synth.decode_workload(shape, 64, seed=1000, in_dtype="f32", ckpt_std=0.0)
    cfg = staging.config(shape, in_dtype="f32")
    say("decode tiny f32 (1,4,16,16,1) L=4 64 steps")
    y, st, p = run_decode(cfg, work, 64, dev)
    yref, Href = orc_mod.decode(work)
    assert_rows_close(y, yref, what="tiny decode outputs")
    # 64 tokens with L=4 and fold-at-start: 15 flushes of 4, 4 records pending
    meta = host(st.meta)
    assert np.all(meta[0, :, 1] == 4) and np.all(meta[0, :, 0] == (60 % cfg.cap))
    say("flush tiny")
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    assert np.all(host(st.meta)[0, :, 1] == 0)
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0


@pytest.mark.parametrize("batch,n0", [(3, "steady"), (16, "steady"), (16, "staggered"), (9, 0)])
def test_decode_nemotron_small_batch(batch, n0):
    """Nemotron-3 layer shape (128 heads, 64x128 tiles, 8 groups), bf16 inputs, L=16."""
    dev = device()
    shape = synth.LayerShape(batch=batch, window=16, **NEMO)
    fill = {"steady": 16, "staggered": synth.staggered_fill(batch, 16), 0: 0}[n0]
    work = synth.decode_workload(shape, 40, seed=1001, n0=fill)
    cfg = staging.config(shape)
    say(f"decode nemotron batch={batch} n0={n0} 40 steps")
    y, st, p = run_decode(cfg, work, 40, dev)
    yref, Href = orc_mod.decode(work)
    assert_rows_close(y, yref, what=f"decode outputs batch={batch} n0={n0}")
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0


def test_decode_full_batch_sampled():
    """Full headline layer (batch 256, L=16, steady state), 64 steps; oracle on 4 sequences."""
    dev = device()
    shape = synth.NEMOTRON3
    work = synth.decode_workload(shape, 64, seed=1001, n0=16)
    cfg = staging.config(shape)
    say("decode full batch 256, 64 steps")
    y, st, p = run_decode(cfg, work, 64, dev)
    seqs = np.array([0, 77, 128, 255])
    yref, _ = orc_mod.decode(work, seqs=seqs)
    assert_rows_close(y[:, seqs], yref, what="full-batch decode outputs (sampled)")
    meta = host(st.meta)
    # 16 committed + 64 tokens: flushes at tokens 1, 17, 33, 49 -> 16 records pending
    assert np.all(meta[:, :, 1] == 16)
    assert np.all(np.isfinite(y))


def test_conventional_matches_oracle():
    dev = device()
    for shape, in_dtype, steps, seqs in [
        (synth.TINY, "f32", 64, None),
        (synth.LayerShape(batch=5, window=16, **NEMO), "bf16", 24, None),
        (synth.NEMOTRON3, "bf16", 8, np.array([1, 200])),
    ]:
        work = synth.decode_workload(shape, steps, seed=1002, in_dtype=in_dtype,
                                     ckpt_std=0.0 if shape is synth.TINY else 0.1)
        cfg = staging.config(shape, in_dtype=in_dtype)
        states = staging.conventional_states(cfg, work.h0, 1, dev)
        p = staging.params(work, dev)
        stream = staging.TokenStream(work.steps, dev)
        y = torch.empty((steps, cfg.batch, 1, cfg.nheads, cfg.headdim), device=dev)
        say(f"conventional batch={shape.batch} hd={shape.headdim} steps={steps}")
        for t in range(steps):
            rb.conventional_state_update(cfg, states, p, stream.call(t), y[t])
        torch.cuda.synchronize()
        yref, Href = orc_mod.decode(work, seqs=seqs)
        sl = slice(None) if seqs is None else seqs
        assert_rows_close(host(y)[:, sl, 0], yref, what="conventional outputs")
        assert tile_err(host(states)[sl, 0], Href).max() <= TOL


@pytest.mark.parametrize("batch,rounds", [(7, 24), (64, 10)])
def test_verify_commit_matches_oracle(batch, rounds):
    """T=3 drafts per round, accepted ~ U{0..3}: outputs of all drafts and the state
    after committing only the accepted ones."""
    dev = device()
    T = 3
    shape = synth.LayerShape(batch=batch, window=16, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, rounds, T, seed=1003)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, batch, T, cfg.nheads, cfg.headdim), device=dev)
    say(f"verify T=3 batch={batch} rounds={rounds}")
    for r in range(rounds):
        rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
        rb.replayssm_commit(cfg, st, acc[r], T)
    torch.cuda.synchronize()
    yref, Href = orc_mod.verify_rounds(work)
    # yref [rounds][T][batch][nh][hd] vs y [rounds][batch][T][nh][hd]
    assert_rows_close(np.swapaxes(host(y), 1, 2), yref, what="verify outputs")
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0


SHAPES = {
    "16x16": dict(nheads=4, headdim=16, dstate=16, ngroups=1),
    "64x64": dict(nheads=16, headdim=64, dstate=64, ngroups=2),
    "64x128": NEMO,
    "128x128": dict(nheads=8, headdim=128, dstate=128, ngroups=1),
}


@pytest.mark.parametrize("tile,in_dtype,L,T,batch,rounds", [
    ("16x16", "f32", 4, 8, 3, 12),       # most drafts, window shorter than the drafts
    ("64x64", "bf16", 16, 4, 3, 12),
    ("128x128", "f32", 8, 2, 3, 16),
    ("64x128", "bf16", 16, 8, 4, 10),     # most drafts at the layer shape
    ("64x128", "bf16", 64, 4, 3, 40),     # longest window at the layer shape (cap 71)
    ("128x128", "bf16", 32, 3, 2, 24),
])
def test_verify_shapes_and_limits(tile, in_dtype, L, T, batch, rounds):
    """Every compiled tile shape, fp32 and bf16 inputs, up to the largest draft
    count and window: verify + commit outputs and the state after a final flush
    against the oracle stepping through the same drafts."""
    dev = device()
    shape = synth.LayerShape(batch=batch, window=L, max_drafts=T, **SHAPES[tile])
    work = synth.verify_workload(shape, rounds, T, seed=1006, in_dtype=in_dtype)
    cfg = staging.config(shape, in_dtype=in_dtype)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, batch, T, cfg.nheads, cfg.headdim), device=dev)
    say(f"verify {tile} {in_dtype} L={L} T={T} batch={batch} rounds={rounds}")
    for r in range(rounds):
        rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
        rb.replayssm_commit(cfg, st, acc[r], T)
    torch.cuda.synchronize()
    yref, Href = orc_mod.verify_rounds(work)
    assert_rows_close(np.swapaxes(host(y), 1, 2), yref, what=f"verify outputs {tile} L={L} T={T}")
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    assert tile_err(host(st.ckpt), Href).max() <= TOL
    assert host(st.status)[0] == 0


def test_snapshot_baseline_matches_oracle():
    """Conventional speculative baseline: one snapshot per draft, slot-select commit."""
    dev = device()
    T, batch, rounds = 3, 6, 12
    shape = synth.LayerShape(batch=batch, window=16, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, rounds, T, seed=1004, n0=0)
    cfg = staging.config(shape)
    states = staging.conventional_states(cfg, work.h0, T + 1, dev)
    slot = torch.zeros(batch, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, batch, T, cfg.nheads, cfg.headdim), device=dev)
    say("snapshot baseline T=3")
    for r in range(rounds):
        rb.conventional_state_update(cfg, states, p, stream.call(r), y[r], slot=slot, status=status)
        rb.conventional_commit(cfg, slot, T + 1, acc[r], T, status=status)
    torch.cuda.synchronize()
    yref, Href = orc_mod.verify_rounds(work)
    assert_rows_close(np.swapaxes(host(y), 1, 2), yref, what="snapshot verify outputs")
    s = host(slot)
    final = host(states)[np.arange(batch), s]
    assert tile_err(final, Href).max() <= TOL
    assert host(status)[0] == 0


def test_decode_equals_verify1_commit1_bitwise():
    """decode_step is verify_drafts(T=1) followed by commit(1): identical bits."""
    dev = device()
    shape = synth.LayerShape(batch=4, window=4, max_drafts=1, **NEMO)
    work = synth.decode_workload(shape, 11, seed=1005, n0=2)
    cfg = staging.config(shape)
    st1 = staging.replay_state(cfg, work, dev)
    st2 = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev)
    ones = torch.ones(shape.batch, dtype=torch.int32, device=dev)
    y1 = torch.empty((shape.batch, 1, cfg.nheads, cfg.headdim), device=dev)
    y2 = torch.empty_like(y1)
    say("decode vs verify(1)+commit(1)")
    for t in range(11):
        rb.replayssm_decode_step(cfg, st1, p, stream.call(t), y1)
        rb.replayssm_verify_drafts(cfg, st2, p, stream.call(t), y2)
        rb.replayssm_commit(cfg, st2, ones, 1)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        assert torch.equal(st1.meta, st2.meta)
    assert torch.equal(st1.ckpt, st2.ckpt)


def test_records_beyond_pointer_are_ignored():
    """NaN-poison every ring slot past the committed records before each call:
    outputs stay finite and bit-identical to an unpoisoned run."""
    dev = device()
    T = 2
    shape = synth.LayerShape(batch=5, window=6, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, 14, T, seed=1006)
    cfg = staging.config(shape)
    clean = staging.replay_state(cfg, work, dev)
    dirty = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y1 = torch.empty((shape.batch, T, cfg.nheads, cfg.headdim), device=dev)
    y2 = torch.empty_like(y1)
    nan_bf16 = torch.tensor(float("nan"), dtype=torch.bfloat16)
    say("NaN-poisoned slots past the pointer")
    for r in range(14):
        meta = host(dirty.meta)
        for b in range(shape.batch):
            start, n = int(meta[b, 0, 0]), int(meta[b, 0, 1])
            for k in range(n, cfg.cap):
                s = (start + k) % cfg.cap
                dirty.buf_x[b, :, s] = nan_bf16
                dirty.buf_B[b, :, s] = nan_bf16
                dirty.buf_dt[b, :, s] = float("nan")
        rb.replayssm_verify_drafts(cfg, clean, p, stream.call(r), y1)
        rb.replayssm_verify_drafts(cfg, dirty, p, stream.call(r), y2)
        rb.replayssm_commit(cfg, clean, acc[r], T)
        rb.replayssm_commit(cfg, dirty, acc[r], T)
        torch.cuda.synchronize()
        assert torch.isfinite(y2).all()
        assert torch.equal(y1, y2)
    assert torch.equal(clean.ckpt, dirty.ckpt)


def test_bad_meta_and_accept_set_status():
    """A corrupt ring pointer or an accepted count > T is reported, not applied."""
    dev = device()
    shape = synth.LayerShape(batch=3, window=4, max_drafts=2, **NEMO)
    work = synth.decode_workload(shape, 1, seed=1007, n0=1)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    tok = staging.tokens_block(work.steps, 0, 1, dev)
    st.meta[1, :, 1] = cfg.cap + 3   # sequence 1 corrupt
    y = torch.zeros((3, 1, cfg.nheads, cfg.headdim), device=dev)
    say("corrupt meta")
    rb.replayssm_decode_step(cfg, st, p, tok, y)
    torch.cuda.synchronize()
    assert host(st.status)[0] & rb.RSSM_STATUS_META
    assert torch.isnan(y[1]).all() and torch.isfinite(y[0]).all() and torch.isfinite(y[2]).all()
    meta = host(st.meta)
    assert np.all(meta[1, :, 1] == cfg.cap + 3) and np.all(meta[0, :, 1] == 2) and np.all(meta[2, :, 1] == 2)
    st.status.zero_()
    st.meta[1, :, 1] = 1
    acc = torch.tensor([0, 5, 1], dtype=torch.int32, device=dev)
    rb.replayssm_commit(cfg, st, acc, 2)
    torch.cuda.synchronize()
    assert host(st.status)[0] & rb.RSSM_STATUS_ACCEPT
    assert np.all(host(st.meta)[:, :, 1] == np.array([2, 1, 3])[:, None])


def test_zero_batch_is_noop():
    dev = device()
    cfg = rb.Config(0, 128, 64, 128, 8, 16, 1)
    st = rb.State.allocate(cfg, dev)
    p = rb.Params(torch.zeros(128, device=dev), torch.zeros(128, device=dev))
    tok = rb.Tokens(torch.zeros((0, 1, 128, 64), dtype=torch.bfloat16, device=dev),
                    torch.zeros((0, 1, 8, 128), dtype=torch.bfloat16, device=dev),
                    torch.zeros((0, 1, 8, 128), dtype=torch.bfloat16, device=dev),
                    torch.zeros((0, 1, 128), device=dev))
    y = torch.zeros((0, 1, 128, 64), device=dev)
    rb.replayssm_decode_step(cfg, st, p, tok, y)
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()


def test_commit_verify_equals_commit_then_verify_bitwise():
    """replayssm_commit_verify(a_prev, drafts) == commit(a_prev) then verify_drafts(drafts)."""
    dev = device()
    T, rounds = 3, 20
    shape = synth.LayerShape(batch=6, window=8, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, rounds, T, seed=1008)
    cfg = staging.config(shape)
    st1 = staging.replay_state(cfg, work, dev)
    st2 = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y1 = torch.empty((shape.batch, T, cfg.nheads, cfg.headdim), device=dev)
    y2 = torch.empty_like(y1)
    say("commit_verify vs commit + verify")
    for r in range(rounds):
        if r == 0:
            rb.replayssm_verify_drafts(cfg, st1, p, stream.call(r), y1)
            rb.replayssm_verify_drafts(cfg, st2, p, stream.call(r), y2)
        else:
            rb.replayssm_commit(cfg, st1, acc[r - 1], T)
            rb.replayssm_verify_drafts(cfg, st1, p, stream.call(r), y1)
            rb.replayssm_commit_verify(cfg, st2, p, acc[r - 1], T, stream.call(r), y2)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"round {r}"
        assert torch.equal(st1.meta, st2.meta), f"round {r}"
    rb.replayssm_commit(cfg, st1, acc[rounds - 1], T)
    rb.replayssm_commit(cfg, st2, acc[rounds - 1], T)
    rb.replayssm_flush(cfg, st1, p)
    rb.replayssm_flush(cfg, st2, p)
    torch.cuda.synchronize()
    assert torch.equal(st1.ckpt, st2.ckpt) and torch.equal(st1.meta, st2.meta)
    assert host(st1.status)[0] == 0 and host(st2.status)[0] == 0


def test_commit_verify_rejects_bad_accepted_count():
    dev = device()
    T = 2
    shape = synth.LayerShape(batch=3, window=4, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, 1, T, seed=1009, n0=1)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    tok = staging.TokenStream(work.steps, dev, T=T).call(0)
    y = torch.zeros((3, T, cfg.nheads, cfg.headdim), device=dev)
    say("commit_verify with accepted > T")
    rb.replayssm_commit_verify(cfg, st, p, torch.tensor([1, 3, 0], dtype=torch.int32, device=dev), T, tok, y)
    torch.cuda.synchronize()
    assert host(st.status)[0] & rb.RSSM_STATUS_ACCEPT
    assert torch.isnan(y[1]).all() and torch.isfinite(y[0]).all() and torch.isfinite(y[2]).all()
    meta = host(st.meta)
    assert np.all(meta[0, :, 1] == 2) and np.all(meta[1, :, 1] == 1) and np.all(meta[2, :, 1] == 1)


@pytest.mark.parametrize("read_copy", [None, "e4m3"])
def test_rollback_equals_decoding_the_accepted_prefix(read_copy):
    """verify(T drafts) + commit(a) + K decode steps on one state; on a second
    state, only the accepted drafts are stepped (one draft per launch, the
    rejected ones rolled back by committing 0 of them), then the same K steps.
    The K steps' outputs and the final checkpoints agree within 1e-6 of their
    scale (the two paths fold at different moments, so only rounding differs);
    accepted counts differ per sequence, 0 .. T."""
    dev = device()
    T, L, K = 4, 6, 13
    batch = T + 1
    shape = synth.LayerShape(batch=batch, window=L, max_drafts=T, **NEMO)
    work = synth.decode_workload(shape, T + K, seed=1016, n0=synth.staggered_fill(batch, L))
    cfg = staging.config(shape, read_copy=read_copy)
    p = staging.params(work, dev)
    accepted = np.arange(batch, dtype=np.int32) % (T + 1)                 # 0, 1, .., T
    drafts = staging.tokens_block(work.steps, 0, T, dev)
    later = staging.TokenStream(work.steps.slice(T, T + K), dev)
    say(f"rollback vs accepted-prefix decode, copy={read_copy}")

    def finish(st):
        y = torch.empty((K, batch, 1, shape.nheads, shape.headdim), device=dev)
        for t in range(K):
            rb.replayssm_decode_step(cfg, st, p, later.call(t), y[t])
        rb.replayssm_flush(cfg, st, p)
        torch.cuda.synchronize()
        assert int(host(st.status)[0]) == 0
        return host(y)[:, :, 0], host(st.ckpt)

    st_a = staging.replay_state(cfg, work, dev)
    if read_copy:
        rb.replayssm_flush(cfg, st_a, p, rb.RSSM_FLUSH_FORCE_CAST)
    ya = torch.empty((batch, T, shape.nheads, shape.headdim), device=dev)
    rb.replayssm_verify_drafts(cfg, st_a, p, drafts, ya)
    rb.replayssm_commit(cfg, st_a, torch.from_numpy(accepted).to(dev), T)
    y_a, h_a = finish(st_a)

    st_b = staging.replay_state(cfg, work, dev)
    if read_copy:
        rb.replayssm_flush(cfg, st_b, p, rb.RSSM_FLUSH_FORCE_CAST)
    one = staging.TokenStream(work.steps.slice(0, T), dev)
    yb = torch.empty((batch, 1, shape.nheads, shape.headdim), device=dev)
    for j in range(T):
        rb.replayssm_verify_drafts(cfg, st_b, p, one.call(j), yb)
        rb.replayssm_commit(cfg, st_b, torch.from_numpy((j < accepted).astype(np.int32)).to(dev), 1)
    y_b, h_b = finish(st_b)

    assert np.all(host(st_a.meta)[:, :, 1] == 0) and np.all(host(st_b.meta)[:, :, 1] == 0)
    scale = np.abs(y_b).max(axis=(0, 3))
    err = np.abs(y_a - y_b).max(axis=(0, 3)) / scale
    print(f"[gpu] rollback: max output difference {err.max():.2e} of scale", flush=True)
    assert err.max() <= 1e-6
    assert tile_err(h_a, h_b).max() <= 1e-6


def test_verify_full_batch_sampled():
    """The benchmarked verification workload (batch 512, T = 3 drafts,
    accepted U{0..3}, L = 16, initial fill U{0..15}, the bench's seed), 12
    rounds through the fused commit + verify entry point: sampled sequences'
    draft outputs and, after the last commit and a flush, their state."""
    dev = device()
    T, rounds = 3, 12
    shape = synth.LayerShape(batch=512, window=16, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, rounds, T, seed=1003)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, shape.batch, T, cfg.nheads, cfg.headdim), device=dev)
    say(f"verify full batch 512, T={T}, {rounds} rounds (fused commit)")
    for r in range(rounds):
        if r == 0:
            rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
        else:
            rb.replayssm_commit_verify(cfg, st, p, acc[r - 1], T, stream.call(r), y[r])
    rb.replayssm_commit(cfg, st, acc[rounds - 1], T)
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    seqs = np.array([0, 100, 300, 511])
    yref, Href = orc_mod.verify_rounds(work, seqs=seqs)
    assert_rows_close(np.swapaxes(host(y)[:, seqs], 1, 2), yref, what="full-batch verify outputs (sampled)")
    assert tile_err(host(st.ckpt[torch.from_numpy(seqs).to(dev)]), Href).max() <= TOL
    assert np.all(host(st.meta)[:, :, 1] == 0)
    assert host(st.status)[0] == 0
