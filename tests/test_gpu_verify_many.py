"""GPU parity of verification with several drafts over large launches.

Speculative verification of T = 4 .. 8 drafts per call (NVIDIA Developer blog
"ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding",
section "Benefit 2": one read of the checkpoint serves every draft; Fig. 5 times
T = 8) over launches of more than 512 workgroups (smaller ones take the
small-batch variant): the draft outputs match the fp64 oracle per (sequence,
head, draft) row through flushes inside verification calls, for every compiled
tile shape, both input types and the longest window; degenerate layer
parameters at T = 8; and the benchmarked T = 8 workload at full size through
the fused commit + verify entry point.  A few sequences of each launch are
checked against the oracle.
"""
import math

import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from tests.gpu_util import TOL, assert_rows_close, device, host, say, tile_err
from tests.test_gpu_edges import _degenerate

pytestmark = pytest.mark.gpu

SHAPES = {
    "16x16": dict(nheads=4, headdim=16, dstate=16, ngroups=1),
    "64x64": dict(nheads=16, headdim=64, dstate=64, ngroups=2),
    "64x128": dict(nheads=128, headdim=64, dstate=128, ngroups=8),
    "128x128": dict(nheads=8, headdim=128, dstate=128, ngroups=1),
}


def _batch_over_512_workgroups(nheads):
    return math.ceil(520 / nheads)


def _run(cfg, work, T, dev, fused=False):
    rounds = work.extra["accepted"].shape[0]
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((rounds, cfg.batch, T, cfg.nheads, cfg.headdim), device=dev)
    for r in range(rounds):
        if fused and r > 0:
            rb.replayssm_commit_verify(cfg, st, p, acc[r - 1], T, stream.call(r), y[r])
        else:
            rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
        if not fused:
            rb.replayssm_commit(cfg, st, acc[r], T)
    if fused:
        rb.replayssm_commit(cfg, st, acc[rounds - 1], T)
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    return np.swapaxes(host(y), 1, 2), st


def _seqs(batch):
    return np.unique(np.array([0, 1, batch // 2, batch - 1]))


@pytest.mark.parametrize("tile,in_dtype,L,T,rounds", [
    ("64x128", "f32", 16, 8, 6),
    ("64x128", "bf16", 16, 8, 8),
    ("64x128", "bf16", 16, 4, 8),
    ("64x128", "f32", 4, 5, 8),        # window shorter than the drafts, odd T
    ("64x128", "bf16", 64, 8, 14),     # longest window at the most drafts (ring of 79)
    ("64x64", "bf16", 16, 8, 6),
    ("128x128", "f32", 8, 6, 6),
    ("16x16", "f32", 4, 8, 8),
])
def test_many_drafts_verify_matches_oracle(tile, in_dtype, L, T, rounds):
    dev = device()
    batch = _batch_over_512_workgroups(SHAPES[tile]["nheads"])
    shape = synth.LayerShape(batch=batch, window=L, max_drafts=T, **SHAPES[tile])
    work = synth.verify_workload(shape, rounds, T, seed=1201 + T, in_dtype=in_dtype)
    cfg = staging.config(shape, in_dtype=in_dtype)
    say(f"verify {tile} {in_dtype} L={L} T={T} batch={batch} rounds={rounds}")
    y, st = _run(cfg, work, T, dev)
    seqs = _seqs(batch)
    yref, Href = orc_mod.verify_rounds(work, seqs=seqs)
    assert_rows_close(y[:, :, seqs], yref, what=f"verify outputs {tile} L={L} T={T}")
    assert tile_err(host(st.ckpt)[seqs], Href).max() <= TOL
    assert np.all(host(st.meta)[:, :, 1] == 0)
    assert host(st.status)[0] == 0


@pytest.mark.parametrize("case", ["A0", "dt0", "C0", "strong_decay"])
def test_many_drafts_degenerate_parameters(case):
    """A = 0, dt = 0, C = 0 (every draft output exactly D x: the tile product
    and every score vanish and the one non-zero product is rounded once) and a
    decay that underflows inside the window, at T = 8."""
    dev = device()
    L, T, rounds = 4, 8, 6
    shape = synth.LayerShape(batch=5, window=L, max_drafts=T, **SHAPES["64x128"])
    work = _degenerate(synth.verify_workload(shape, rounds, T, seed=1211), case)
    cfg = staging.config(shape)
    say(f"verify with {case}, L={L}, T={T}")
    y, st = _run(cfg, work, T, dev)
    seqs = np.array([0, 4])
    yref, Href = orc_mod.verify_rounds(work, seqs=seqs)
    assert_rows_close(y[:, :, seqs], yref, what=f"verify outputs ({case}, T=8)")
    assert tile_err(host(st.ckpt)[seqs], Href).max() <= TOL
    assert host(st.status)[0] == 0
    if case == "C0":
        x = work.steps.x.reshape((rounds, T) + work.steps.x.shape[1:])
        want = work.D.astype(np.float32)[None, None, None, :, None] * x.astype(np.float32)
        assert np.array_equal(y, want), "C = 0: the draft outputs are not exactly D x"
    if case == "dt0":
        assert np.array_equal(host(st.ckpt), work.h0)


def test_many_drafts_full_batch_sampled():
    """The benchmarked verification workload at T = 8 (batch 512, accepted
    U{0..8}, L = 16, initial fill U{0..15}, the bench's seed), 6 rounds through
    the fused commit + verify entry point: sampled sequences' draft outputs and,
    after the last commit and a flush, their state."""
    dev = device()
    T, rounds = 8, 6
    shape = synth.LayerShape(batch=512, window=16, max_drafts=T, **SHAPES["64x128"])
    work = synth.verify_workload(shape, rounds, T, seed=1003)
    cfg = staging.config(shape)
    say(f"verify, full batch 512, T={T}, {rounds} rounds (fused commit)")
    y, st = _run(cfg, work, T, dev, fused=True)
    seqs = np.array([0, 100, 300, 511])
    yref, Href = orc_mod.verify_rounds(work, seqs=seqs)
    assert_rows_close(y[:, :, seqs], yref, what="full-batch T=8 verify outputs (sampled)")
    assert tile_err(host(st.ckpt[torch.from_numpy(seqs).to(dev)]), Href).max() <= TOL
    assert np.all(host(st.meta)[:, :, 1] == 0)
    assert host(st.status)[0] == 0
