"""Decode and verify launches captured in a HIP graph (through torch.cuda.graph):
every replay must reproduce, bit for bit, the eager launches of the same
tokens on the same state.  The library's entry points allocate nothing and
issue only kernel launches on the caller's stream, so they can be captured;
this checks it.  Each replay is separated by eager work and a synchronisation,
and compared on its own.  With an FP16 checkpoint the stochastic rounding's
seed is set per step before each call, the same in the captured and the eager
launches, so the rounding is reproduced bit for bit as well."""
import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from tests.gpu_util import device, host, say

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)


def _clone(st: rb.State) -> rb.State:
    return rb.State(**{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in vars(st).items()})


CKPTS = [("f32", None), ("f16", None), ("f16", "mxfp4")]


@pytest.mark.parametrize("ckpt,copy", CKPTS)
def test_decode_graph_replays_match_eager(ckpt, copy):
    dev = device()
    L, K = 4, 10                      # 10 steps per replay: flushes inside the graph
    shape = synth.LayerShape(batch=8, window=L, **NEMO)
    work = synth.decode_workload(shape, K, seed=1013, n0=synth.staggered_fill(8, L))
    cfg = staging.config(shape, read_copy=copy, ckpt_dtype=ckpt)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev)
    st_e = staging.replay_state(cfg, work, dev)
    if copy:
        rb.replayssm_flush(cfg, st_e, p, rb.RSSM_FLUSH_FORCE_CAST)
    st_g = _clone(st_e)
    y_e = torch.empty((K, 8, 1, 128, 64), device=dev)
    y_g = torch.empty((K, 8, 1, 128, 64), device=dev)
    say(f"capture 10 decode steps, {ckpt} checkpoint, copy {copy}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(K):
            p.sr_seed = 500 + t
            rb.replayssm_decode_step(cfg, st_g, p, stream.call(t), y_g[t])
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"eager pass {rep}")
        for t in range(K):
            p.sr_seed = 500 + t
            rb.replayssm_decode_step(cfg, st_e, p, stream.call(t), y_e[t])
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        y_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}: outputs differ from the eager launches"
        assert torch.equal(st_g.ckpt, st_e.ckpt) and torch.equal(st_g.meta, st_e.meta)
        if copy:
            assert torch.equal(st_g.ckpt_read, st_e.ckpt_read) and torch.equal(st_g.ckpt_scale, st_e.ckpt_scale)
        assert torch.equal(st_g.buf_x, st_e.buf_x) and torch.equal(st_g.buf_B, st_e.buf_B)
    assert int(host(st_g.status)[0]) == 0


@pytest.mark.parametrize("ckpt,copy", CKPTS)
def test_verify_commit_graph_replays_match_eager(ckpt, copy):
    dev = device()
    T, L, R = 3, 8, 4
    shape = synth.LayerShape(batch=6, window=L, max_drafts=T, **NEMO)
    work = synth.verify_workload(shape, R, T, seed=1014)
    cfg = staging.config(shape, read_copy=copy, ckpt_dtype=ckpt)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    st_e = staging.replay_state(cfg, work, dev)
    if copy:
        rb.replayssm_flush(cfg, st_e, p, rb.RSSM_FLUSH_FORCE_CAST)
    st_g = _clone(st_e)
    y_e = torch.empty((R, 6, T, 128, 64), device=dev)
    y_g = torch.empty((R, 6, T, 128, 64), device=dev)
    say(f"capture 4 verify + commit rounds, {ckpt} checkpoint, copy {copy}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            p.sr_seed = 900 + r
            rb.replayssm_verify_drafts(cfg, st_g, p, stream.call(r), y_g[r])
            rb.replayssm_commit(cfg, st_g, acc[r], T)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"eager pass {rep}")
        for r in range(R):
            p.sr_seed = 900 + r
            rb.replayssm_verify_drafts(cfg, st_e, p, stream.call(r), y_e[r])
            rb.replayssm_commit(cfg, st_e, acc[r], T)
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        y_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}: outputs differ from the eager launches"
        assert torch.equal(st_g.ckpt, st_e.ckpt) and torch.equal(st_g.meta, st_e.meta)
        if copy:
            assert torch.equal(st_g.ckpt_read, st_e.ckpt_read) and torch.equal(st_g.ckpt_scale, st_e.ckpt_scale)
    assert int(host(st_g.status)[0]) == 0
