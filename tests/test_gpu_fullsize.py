"""Parity at the full sizes the benchmark times, in the same launch
configuration, on sampled sequences (the fp64 oracle runs a handful of
sequences; every sequence's outputs are checked finite):

* speculative verification, batch 512, T = 3, accepted U{0..T}, verify then
  commit as the benchmark issues them (and the fused commit);
* decode at the largest batch of the sweep and at the shortest and longest
  windows;
* the read copies at batch 256, L = 16: outputs of non-flush steps within the
  copy's per-element read bound of the oracle, the FP32 checkpoint
  bit-identical to an FP32-only run.
"""
import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from tests import formats
from tests.gpu_util import TOL, assert_rows_close, device, host, say

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)


@pytest.mark.parametrize("fused", [False, True])
def test_verify_batch512_t3_sampled(fused):
    dev = device()
    T, rounds = 3, 14                                   # about 21 accepted tokens: every sequence flushes once
    shape = synth.LayerShape(batch=512, window=16, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, rounds, T, seed=1003)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, 512, T, 128, 64), device=dev)
    say(f"verify batch 512 T=3, {rounds} rounds, fused commit {fused}")
    for r in range(rounds):
        if fused and r > 0:
            rb.replayssm_commit_verify(cfg, st, p, acc[r - 1], T, stream.call(r), y[r])
        else:
            rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
            if not fused:
                rb.replayssm_commit(cfg, st, acc[r], T)
    if fused:
        rb.replayssm_commit(cfg, st, acc[rounds - 1], T)
    torch.cuda.synchronize()
    yg = host(y)
    assert np.all(np.isfinite(yg)) and int(host(st.status)[0]) == 0
    seqs = np.array([0, 131, 300, 511])
    yref, _ = orc_mod.verify_rounds(work, seqs=seqs)
    assert_rows_close(np.swapaxes(yg[:, seqs], 1, 2), yref, what="batch-512 verify outputs (sampled)")


@pytest.mark.parametrize("batch,L", [(512, 16), (256, 4), (256, 32)])
def test_decode_sweep_points_sampled(batch, L):
    dev = device()
    steps = 2 * L + 3
    shape = synth.LayerShape(batch=batch, window=L, **NEMO)
    work = synth.decode_workload(shape, steps, seed=1002, n0=L)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev)
    y = torch.empty((steps, batch, 1, 128, 64), device=dev)
    say(f"decode batch {batch} L={L}, {steps} steps")
    for t in range(steps):
        rb.replayssm_decode_step(cfg, st, p, stream.call(t), y[t])
    torch.cuda.synchronize()
    yg = host(y)[:, :, 0]
    assert np.all(np.isfinite(yg))
    seqs = np.array([0, batch // 3, batch - 1])
    yref, _ = orc_mod.decode(work, seqs=seqs)
    assert_rows_close(yg[:, seqs], yref, what=f"batch {batch} L={L} decode outputs (sampled)")


UNIT = {"bf16": 2.0 ** -8, "e4m3": 2.0 ** -4, "mxfp4": 2.0 ** -2, "mxfp8": 2.0 ** -4}


def _delta(copy, scale):
    """Absolute part of the per-element read bound for one sequence's scales."""
    if copy == "bf16":
        return 0.0
    if copy == "e4m3":
        return (np.asarray(scale, np.float64) * 2.0 ** -10 * 1.001)[:, None, None]
    X = np.repeat(formats.e8m0_value(scale), 32, axis=-1)
    return X * (2.0 ** -10 if copy == "mxfp8" else 0.25) * 1.001


def test_read_copies_batch256_sampled():
    dev = device()
    L, steps = 16, 40
    shape = synth.LayerShape(batch=256, window=L, **NEMO)
    work = synth.decode_workload(shape, steps, seed=1004, n0=L)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev)
    seqs = np.array([3, 128, 254])
    # oracle: H_s at each flush (steps 0, L, 2L flush first) and the outputs
    yref, _ = orc_mod.decode(work, seqs=seqs)
    hs = {0: orc_mod.committed_state(work, seqs=seqs)}
    tok = work.steps
    for tf in range(L, steps, L):
        x, B, C, dt = (a[:tf, seqs] for a in (tok.x, tok.B, tok.C, tok.dt))
        hs[tf], _ = orc_mod.conventional(hs[0], x, B, C, dt, work.A, work.D, outputs=False)
    cfg32 = staging.config(shape)
    st32 = staging.replay_state(cfg32, work, dev)
    say("batch 256 FP32 reference run")
    for t in range(steps):
        rb.replayssm_decode_step(cfg32, st32, p, stream.call(t), torch.empty((256, 1, 128, 64), device=dev))
    A = work.A.astype(np.float64)
    hpg = 16
    for copy in ("bf16", "e4m3", "mxfp4", "mxfp8"):
        cfg = staging.config(shape, read_copy=copy)
        st = staging.replay_state(cfg, work, dev)
        y = torch.empty((steps, 256, 1, 128, 64), device=dev)
        scales = {}
        say(f"batch 256 decode with a {copy} copy, {steps} steps")
        for t in range(steps):
            rb.replayssm_decode_step(cfg, st, p, stream.call(t), y[t])
            if t % L == 0 and copy != "bf16":
                scales[t] = host(st.ckpt_scale)[seqs]
        torch.cuda.synchronize()
        assert torch.equal(st.ckpt, st32.ckpt), f"{copy}: the copy changed the FP32 recurrence"
        yg = host(y)[:, :, 0]
        assert np.all(np.isfinite(yg))
        ys = yg[:, seqs].astype(np.float64)
        out_scale = np.abs(yref).max(axis=(0, 3))
        worst = 0.0
        for tf in hs:
            flush_rows = ys[tf] - yref[tf]                 # flushing steps read FP32 registers
            assert float((np.abs(flush_rows).max(axis=-1) / out_scale).max()) <= TOL
            for t in range(tf + 1, min(tf + L, steps)):
                dec = np.exp(A[None, :] * tok.dt[tf:t + 1, seqs].astype(np.float64).sum(0))
                Cg = np.repeat(np.abs(tok.C[t, seqs].astype(np.float64)), hpg, axis=1)
                term = UNIT[copy] * np.abs(hs[tf]) + _delta(copy, scales.get(tf))
                bound = dec[:, :, None] * np.einsum("bhij,bhj->bhi", term, Cg) + TOL * out_scale[:, :, None]
                worst = max(worst, float((np.abs(ys[t] - yref[t]) / bound).max()))
        print(f"[gpu] batch 256 {copy}: worst error/bound {worst:.3f}", flush=True)
        assert worst <= 1.0
        del st
        torch.cuda.empty_cache()
