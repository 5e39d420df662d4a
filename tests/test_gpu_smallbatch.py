"""The small-batch launch: at 512 workgroups or fewer an FP32-reading call
issues the loads of every ring slot, of its tokens, dt and the FP32 tile before
its ring pointer arrives (the eager variant), then routes the vectors it needs
to their window rows.  It must equal the streaming launch bit for bit: each
output row and each state element is computed by the same lanes from the same
values in the same order either way.
"""
import dataclasses

import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from tests.gpu_util import assert_rows_close, device, host, say

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)


def _first_sequences(work: synth.Workload, k: int) -> synth.Workload:
    """The same workload restricted to its first k sequences."""
    def tok(t):
        cut = lambda a: None if a is None else a[:, :k]
        return synth.Tokens(t.x[:, :k], t.B[:, :k], t.C[:, :k], t.dt[:, :k], t.in_dtype,
                            cut(t.x_bits), cut(t.B_bits), cut(t.C_bits))
    extra = dict(work.extra)
    if "accepted" in extra:
        extra["accepted"] = extra["accepted"][:, :k]
    return dataclasses.replace(work, shape=dataclasses.replace(work.shape, batch=k), h0=work.h0[:k],
                               n0=work.n0[:k], pre=tok(work.pre), steps=tok(work.steps), extra=extra)


@pytest.mark.parametrize("L,T", [(4, 3), (16, 1), (32, 2)])
def test_eager_small_batch_equals_streaming_launch(L, T):
    """At 512 workgroups or fewer an FP32-reading call loads every ring slot,
    the tokens and the tile before its ring pointer arrives (the eager
    variant); at 5 sequences x 128 heads it streams as usual.  The first 4
    sequences of a 5-sequence run and the same 4 sequences run alone (eager)
    give bit-identical outputs, checkpoints and pointers through flushes,
    verification and rollback."""
    dev = device()
    rounds = 12
    shape = synth.LayerShape(batch=5, window=L, max_drafts=T, **NEMO)
    w5 = synth.verify_workload(shape, rounds, T, seed=1206)
    w4 = _first_sequences(w5, 4)
    res = {}
    for name, work in (("streaming", w5), ("eager", w4)):
        cfg = staging.config(work.shape)
        st = staging.replay_state(cfg, work, dev)
        p = staging.params(work, dev)
        stream = staging.TokenStream(work.steps, dev, T=T)
        acc = torch.from_numpy(work.extra["accepted"]).to(dev)
        y = torch.empty((rounds, work.shape.batch, T, 128, 64), device=dev)
        say(f"{name} launch, batch {work.shape.batch}, L={L}, T={T}")
        for r in range(rounds):
            if T == 1 and r % 2 == 0:
                rb.replayssm_decode_step(cfg, st, p, stream.call(r), y[r])
            else:
                rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y[r])
                rb.replayssm_commit(cfg, st, acc[r], T)
        rb.replayssm_flush(cfg, st, p)
        torch.cuda.synchronize()
        assert host(st.status)[0] == 0
        res[name] = (host(y), host(st.ckpt), host(st.meta), host(st.buf_dt))
    ys, cs, ms, ds = res["streaming"]
    ye, ce, me, de = res["eager"]
    assert np.array_equal(ys[:, :4], ye)
    assert np.array_equal(cs[:4], ce)
    assert np.array_equal(ms[:4], me)
    yref, _ = orc_mod.verify_rounds(w4) if T > 1 else (None, None)
    if yref is not None:
        assert_rows_close(np.swapaxes(ye, 1, 2), yref, what=f"eager verify outputs L={L} T={T}")
