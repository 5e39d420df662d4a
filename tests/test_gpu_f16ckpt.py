"""GPU tests of the FP16 recurrence checkpoint written with stochastic rounding
(NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
Hybrid-Model Decoding", section "Benefit 3: Limit error accumulation with
separate precisions": a half-precision recurrence state stays close to FP32 when
its writes round stochastically).

* the kernel's rounding, through the probe entry point, equals the host
  definition (oracle/sr.py) bit for bit;
* a flush writes the stochastic rounding of the exact fold: the same fp16
  value as the oracle for all but the elements whose fp32 value sits at a
  rounding threshold, and there a neighbouring one;
* decoding through several flushes equals the oracle that composes the same
  flush schedule on its own state (exact fold, then stochastic rounding with
  the call's seed) to the FP32 tolerance per row, plus what one fp16 spacing
  per checkpoint element (where a rounding decision went the other way) can
  move an output;
* with an MXFP4 read copy the fp16 checkpoints are bit-identical to a run
  without one, and the outputs stay within the copy's read bound of that
  oracle;
* where every flush moves the state by less than half an fp16 spacing,
  round-to-nearest stagnates while the stochastic checkpoint tracks the
  exact state (mean error near zero).
"""
import dataclasses

import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from oracle import sr
from tests import formats
from tests.gpu_util import TOL, assert_rows_close, device, host, row_norm, say

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)


def _bits_equal(gpu_f16: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """fp16 results equal to float64 references on the fp16 grid (NaN == NaN)."""
    want = ref.astype(np.float16)
    same = gpu_f16.view(np.uint16) == want.view(np.uint16)
    return same | (np.isnan(gpu_f16) & np.isnan(ref))


def test_sr_probe_matches_host_definition():
    dev = device()
    g = np.random.default_rng(41)
    n = 1 << 22
    parts = [
        np.exp(g.uniform(np.log(2.0 ** -14), np.log(65504.0), n // 2)),          # fp16 normal range
        g.uniform(0, 2.0 ** -14, n // 8),                                          # fp16 subnormal range
        np.exp(g.uniform(-120, -30, n // 16)),                                     # far below
        g.uniform(60000, 70000, n // 16),                                          # saturation
        np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float64),  # the fp16 grid
        [0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 2.0 ** -14, 2.0 ** -24, 1.5 * 2.0 ** -24],
    ]
    v = np.concatenate([np.asarray(p, np.float64) for p in parts])
    v = (v * g.choice([-1.0, 1.0], v.size)).astype(np.float32)
    v = np.concatenate([v, g.standard_normal((-v.size) % 4).astype(np.float32)])
    seed = int(g.integers(0, 2 ** 63))
    vec0 = (1 << 33) + 12345                                                       # high counter word in use
    src = torch.from_numpy(v).to(dev)
    dst = torch.empty(v.size, dtype=torch.float16, device=dev)
    say(f"sr probe, {v.size} values")
    rb.rssm_probe_sr_f16(src, dst, vec0, seed)
    torch.cuda.synchronize()
    want = sr.f16_sr(v, sr.words(np.arange(v.size, dtype=np.uint64) + np.uint64(4 * vec0), seed))
    ok = _bits_equal(host(dst), want)
    if not ok.all():
        i = np.flatnonzero(~ok)[:5]
        print(f"[gpu] mismatches at {v[i]} -> got {host(dst)[i]} want {want[i]}", flush=True)
    assert ok.all(), f"{int((~ok).sum())} values rounded differently"


def _f16_work(shape, steps, seed, n0, in_dtype="bf16"):
    """A workload whose initial checkpoint is on the fp16 grid (the values the
    FP16 state holds), so the oracle starts from exactly what the GPU holds."""
    work = synth.decode_workload(shape, steps, seed=seed, in_dtype=in_dtype, n0=n0)
    return dataclasses.replace(work, h0=work.h0.astype(np.float16).astype(np.float32))


def _spacing_allowance(H, C, nheads):
    """Per-output allowance [batch][nheads][headdim] for reading a checkpoint that
    may differ from the oracle's H by one fp16 spacing per element:
    sum_j |C[b, g(h), j]| * 2 * spacing16(|H[b, h, i, j]|).  Where the kernel's
    fp32 fold and the oracle's fp64 fold straddle a rounding threshold the two
    stochastic roundings are neighbours on the fp16 grid (one spacing of the
    larger value's binade, at most twice the spacing at |H|); later folds decay
    that difference (decays are <= 1) and round it again with the same random
    bits, so it never exceeds one spacing.  C is [batch][ngroups][dstate]."""
    _, sp = sr.f16_grid(np.abs(np.asarray(H, np.float64)))
    Cg = np.repeat(np.abs(np.asarray(C, np.float64)), nheads // C.shape[1], axis=1)
    return np.einsum("bhij,bhj->bhi", 2.0 * sp, Cg)


def _window_allowances(C, cks, L, steps, nheads):
    """Allowances [steps][batch][nheads][headdim] for a decode run whose call tf
    (tf a multiple of L) flushes: the calls after tf read the oracle's rounded
    checkpoint cks[tf]; the flushing call tf > 0 folds the previous one,
    cks[tf - L]; call 0 folds the exact initial checkpoint (no allowance)."""
    out = np.zeros((steps,) + cks[0].shape[:3])
    for t in range(steps):
        tf = t - t % L
        H = cks[tf] if t > tf else cks.get(tf - L)
        if H is not None:
            out[t] = _spacing_allowance(H, C[t], nheads)
    return out


# Every compiled tile shape: the flush's generator calls are shared by a thread's
# vectors 16 apart in rows of 32 vectors (64 x 128, 128 x 128) and of 16 vectors
# (64 x 64: the same column of an even row and the next), and taken per vector
# where a thread holds one vector (16 x 16).
TILES = {
    "16x16": dict(nheads=4, headdim=16, dstate=16, ngroups=1),
    "64x64": dict(nheads=16, headdim=64, dstate=64, ngroups=2),
    "64x128": NEMO,
    "128x128": dict(nheads=8, headdim=128, dstate=128, ngroups=1),
}


@pytest.mark.parametrize("tile", sorted(TILES))
def test_flush_writes_the_stochastic_rounding_of_the_fold(tile):
    dev = device()
    shape = synth.LayerShape(batch=3, window=16, **TILES[tile])
    work = _f16_work(shape, 0, 1020, n0=7, in_dtype="bf16" if tile != "16x16" else "f32")
    cfg = staging.config(shape, ckpt_dtype="f16", in_dtype=work.steps.in_dtype)
    st = staging.replay_state(cfg, work, dev)
    seed = 0x5EED0000F16
    p = dataclasses.replace(staging.params(work, dev), sr_seed=seed)
    say(f"f16 checkpoint flush, {tile} tiles, 7 records")
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    got = host(st.ckpt)
    exact = orc_mod.committed_state(work)
    want = sr.sr_checkpoint(exact, seed)
    same = _bits_equal(got, want)
    # every element is one of the fp16 neighbours of its fp32 fold: within one spacing (the larger of
    # the two binades' at a binade edge) of the exact value, plus the fp32 fold's own error (1e-6 of
    # the tile's largest magnitude covers it; it matters only where the fold cancels to near zero)
    g64 = got.astype(np.float64)
    spacing = np.maximum(sr.f16_grid(np.abs(exact))[1], sr.f16_grid(np.abs(g64))[1])
    slack = 1e-6 * np.abs(exact).max(axis=(-1, -2), keepdims=True)
    dev_ = np.abs(g64 - exact) - spacing - slack
    print(f"[gpu] f16 flush: {same.mean():.6f} of elements equal the oracle's rounding; "
          f"largest excess over one spacing {dev_.max():.3g}", flush=True)
    if (dev_ > 0).any():
        i = np.unravel_index(np.argmax(dev_), dev_.shape)
        print(f"[gpu] worst element {i}: got {g64[i]!r} exact {exact[i]!r} oracle {want[i]!r}", flush=True)
    assert (dev_ <= 0).all(), "an element left the fp16 neighbours of its fold"
    assert same.mean() >= 0.999
    assert np.all(host(st.meta)[:, :, 1] == 0)


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_decode_reads_the_f16_checkpoint(in_dtype):
    """Decode through five flushes (calls 0, L, 2L, ... flush first, each with
    its own seed) against the oracle that follows the same schedule on its own
    state: at a flush it folds exactly (fp64), the flushing call's output reads
    that exact fold, and the checkpoint becomes the stochastic rounding of the
    fold with the call's seed (oracle/sr.py); the other calls read that
    checkpoint plus the window's records.  The Mamba-2 recurrence keeps every
    state element separate, so where a rounding decision went the other way
    (the kernel's fp32 fold and the oracle's fp64 fold straddle a threshold)
    the two checkpoints differ by one fp16 spacing at that element only; the
    outputs meet the FP32 tolerance per row plus what such a spacing can move
    them (_spacing_allowance), and the final checkpoints agree on at least
    99.9% of their elements."""
    dev = device()
    L, steps = 8, 40
    shape = synth.LayerShape(batch=4, window=L, **NEMO)
    work = _f16_work(shape, steps, 1021, n0=L, in_dtype=in_dtype)
    cfg = staging.config(shape, in_dtype=in_dtype, ckpt_dtype="f16")
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    toks = staging.TokenStream(work.steps, dev)
    y = torch.empty((steps, 4, 1, 128, 64), device=dev)
    say(f"f16 checkpoint decode, {in_dtype} inputs, {steps} steps")
    for t in range(steps):
        p.sr_seed = 1000 + t
        rb.replayssm_decode_step(cfg, st, p, toks.call(t), y[t])
    torch.cuda.synchronize()
    yg = host(y)[:, :, 0]
    tok = work.steps
    ref = np.zeros(yg.shape)
    cks = {}
    H = orc_mod.committed_state(work)                     # the exact fold of call 0
    for tf in range(0, steps, L):                         # call tf flushes first
        t1 = min(tf + L, steps)
        win = (tok.x[tf:t1], tok.B[tf:t1], tok.C[tf:t1], tok.dt[tf:t1], work.A, work.D)
        _, yx = orc_mod.conventional(H, *win)
        ck = cks[tf] = sr.sr_checkpoint(H, 1000 + tf)
        H, yc = orc_mod.conventional(ck, *win)            # H: the exact fold of the next flush
        ref[tf] = yx[0]
        ref[tf + 1:t1] = yc[1:]
    assert_rows_close(yg, ref, what="f16-checkpoint decode outputs",
                      allowance=_window_allowances(tok.C, cks, L, steps, shape.nheads))
    same = _bits_equal(host(st.ckpt), ck)
    print(f"[gpu] f16 checkpoint after five flushes: {same.mean():.6f} equal to the oracle's", flush=True)
    assert same.mean() >= 0.999


def test_mxfp4_copy_over_an_f16_checkpoint():
    """FP16 recurrence + MXFP4 read copy: the checkpoints are bit-identical to
    an FP16 run without a copy (same seeds: the copy never enters the
    recurrence).  Against the oracle that composes the same flushes and
    rounding on its own state (as in test_decode_reads_the_f16_checkpoint),
    the no-copy run meets the FP32 tolerance, and the copy run's non-flush
    outputs stay within d_q sum_j |C_q[j]| (|H_s| / 4 + X / 4 + 3 fp16
    spacings of H_s) per element, plus the FP32 tolerance of the row: H_s the oracle's rounded checkpoint, X the
    copy's block scale; the copy is cast from the kernel's fp32 fold, which is
    within a spacing of H_s's exact fold where an earlier rounding decision
    went the other way, and H_s is within a spacing of that fold."""
    dev = device()
    L, steps = 8, 40
    shape = synth.LayerShape(batch=3, window=L, **NEMO)
    work = _f16_work(shape, steps, 1022, n0=L)
    p = staging.params(work, dev)
    toks = staging.TokenStream(work.steps, dev)
    runs = {}
    for copy in (None, "mxfp4"):
        cfg = staging.config(shape, read_copy=copy, ckpt_dtype="f16")
        st = staging.replay_state(cfg, work, dev)       # step 0 flushes the L records and casts the copy
        y = torch.empty((steps, 3, 1, 128, 64), device=dev)
        hs, scs = {}, {}
        say(f"f16 checkpoint + {copy} copy, {steps} steps")
        for t in range(steps):
            p.sr_seed = 7000 + t
            rb.replayssm_decode_step(cfg, st, p, toks.call(t), y[t])
            if t % L == 0:
                hs[t] = host(st.ckpt).astype(np.float64)
                if copy:
                    scs[t] = host(st.ckpt_scale)
        torch.cuda.synchronize()
        runs[copy] = (host(y)[:, :, 0].astype(np.float64), hs, scs)
    y16, h16, _ = runs[None]
    yc, hc, scc = runs["mxfp4"]
    for t in h16:
        assert np.array_equal(h16[t], hc[t]), f"step {t}: the copy changed the fp16 recurrence"
    tok = work.steps
    ref = np.zeros(y16.shape)
    cks = {}
    H = orc_mod.committed_state(work)
    for tf in range(0, steps, L):
        t1 = min(tf + L, steps)
        win = (tok.x[tf:t1], tok.B[tf:t1], tok.C[tf:t1], tok.dt[tf:t1], work.A, work.D)
        _, yx = orc_mod.conventional(H, *win)
        cks[tf] = sr.sr_checkpoint(H, 7000 + tf)
        H, yo = orc_mod.conventional(cks[tf], *win)
        ref[tf] = yx[0]
        ref[tf + 1:t1] = yo[1:]
    assert_rows_close(y16, ref, what="f16-checkpoint outputs without a copy",
                      allowance=_window_allowances(tok.C, cks, L, steps, shape.nheads))
    A = work.A.astype(np.float64)
    hpg = shape.nheads // shape.ngroups
    worst = 0.0
    for tf in cks:
        Hs = np.abs(cks[tf])
        _, sp = sr.f16_grid(Hs)
        X = np.repeat(formats.e8m0_value(scc[tf]), 32, axis=-1)
        term = Hs / 4 + X / 4 * 1.001 + 3 * sp
        for t in range(tf + 1, min(tf + L, steps)):
            dec = np.exp(A[None, :] * work.steps.dt[tf:t + 1].astype(np.float64).sum(0))
            Cg = np.repeat(np.abs(work.steps.C[t].astype(np.float64)), hpg, axis=1)
            # plus the FP32 tolerance of the row (the record terms and the skip term
            # are summed in fp32: an output of 100 carries rounding of order 1e-5)
            bound = dec[:, :, None] * np.einsum("bhij,bhj->bhi", term, Cg) + TOL * row_norm(ref[t][None])[0][..., None]
            worst = max(worst, float((np.abs(yc[t] - ref[t]) / bound).max()))
    print(f"[gpu] f16 + mxfp4: worst error/bound {worst:.3f}", flush=True)
    assert worst <= 1.0


def test_stochastic_rounding_tracks_where_nearest_stagnates():
    """Slow decay (A = -1e-4) and small inputs: every flush moves the state by
    less than half an fp16 spacing.  Round-to-nearest (emulated on the host,
    window by window from the exact fold) keeps the initial values; the GPU's
    stochastic checkpoint follows the exact fp64 state with a mean error (over
    all elements) near zero."""
    dev = device()
    L, windows = 16, 64
    steps = L * windows
    b, nh, hd, ds, ng = 1, 8, 64, 128, 8
    g = np.random.default_rng(43)
    h0 = g.uniform(1.0, 1.9, (b, nh, hd, ds)).astype(np.float16).astype(np.float32)
    x = (0.01 * g.standard_normal((steps, b, nh, hd))).astype(np.float32)
    B = (0.01 * g.standard_normal((steps, b, ng, ds))).astype(np.float32)
    C = g.standard_normal((steps, b, ng, ds)).astype(np.float32)
    dt = np.full((steps, b, nh), 0.13, np.float32)
    A = np.full(nh, -1e-4, np.float32)
    D = np.zeros(nh, np.float32)
    cfg = rb.Config(b, nh, hd, ds, ng, window=L, max_drafts=1, in_dtype="f32", ckpt_dtype="f16")
    st = rb.State.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(h0).half())
    p = rb.Params(torch.from_numpy(A).to(dev), torch.from_numpy(D).to(dev))
    xs, Bs, Cs, dts = (torch.from_numpy(a).to(dev) for a in (x, B, C, dt))
    y = torch.empty((b, 1, nh, hd), device=dev)
    say(f"f16 stagnation case, {steps} steps")
    for t in range(steps):
        p.sr_seed = 90000 + t
        rb.replayssm_decode_step(cfg, st, p, rb.Tokens(xs[t:t + 1].transpose(0, 1).contiguous(),
                                                       Bs[t:t + 1].transpose(0, 1).contiguous(),
                                                       Cs[t:t + 1].transpose(0, 1).contiguous(),
                                                       dts[t:t + 1].transpose(0, 1).contiguous()), y)
    p.sr_seed = 99999
    rb.replayssm_flush(cfg, st, p)                        # fold the last window
    torch.cuda.synchronize()
    got = host(st.ckpt).astype(np.float64)
    orc = orc_mod.default()
    exact, _ = orc.conventional(h0, x, B, C, dt, A, D, outputs=False)
    rn = h0.astype(np.float64)
    for w in range(windows):
        s = slice(w * L, (w + 1) * L)
        rn, _ = orc.conventional(rn, x[s], B[s], C[s], dt[s], A, D, outputs=False)
        rn = rn.astype(np.float16).astype(np.float64)     # round to nearest
    _, sp = sr.f16_grid(np.abs(exact))
    e_sr = (got - exact) / sp
    e_rn = (rn - exact) / sp
    print(f"[gpu] stagnation: mean error in fp16 spacings: stochastic {e_sr.mean():+.3f} (rms {np.sqrt((e_sr ** 2).mean()):.2f}), "
          f"nearest {e_rn.mean():+.2f}", flush=True)
    assert abs(e_rn.mean()) > 10                          # the case does stagnate under nearest rounding
    assert abs(e_sr.mean()) < 0.25
    assert np.sqrt((e_sr ** 2).mean()) < 6


def test_f16_checkpoint_full_batch_sampled():
    """The benchmarked layer (batch 256, 128 heads, headdim 64, dstate 128,
    L = 16) with an FP16 checkpoint: 16 decode steps from 16 committed records,
    so call 0 flushes (with its seed) and calls 1 .. 15 read the fp16
    checkpoint.  Sampled sequences: the flushed checkpoint against the
    stochastic rounding of the exact fold at the elements' flat indices in the
    whole checkpoint, call 0's output against the exact fold, and the later
    outputs against the oracle stepped from its own rounded checkpoint."""
    dev = device()
    L, steps = 16, 16
    shape = synth.LayerShape(batch=256, window=L, **NEMO)
    work = _f16_work(shape, steps, 1031, n0=L)
    cfg = staging.config(shape, ckpt_dtype="f16")
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    toks = staging.TokenStream(work.steps, dev)
    y = torch.empty((steps, shape.batch, 1, 128, 64), device=dev)
    seed = 0xF16F00000100
    say("f16 checkpoint decode, batch 256, 16 steps (flush at call 0)")
    for t in range(steps):
        p.sr_seed = seed + t
        rb.replayssm_decode_step(cfg, st, p, toks.call(t), y[t])
        if t == 0:
            sample = np.array([0, 77, 128, 255])
            ck = host(st.ckpt[torch.from_numpy(sample).to(dev)])
    torch.cuda.synchronize()
    exact = orc_mod.committed_state(work, seqs=sample)
    per_seq = 128 * 64 * 128
    idx = (sample.astype(np.uint64)[:, None] * np.uint64(per_seq)
           + np.arange(per_seq, dtype=np.uint64)[None, :]).reshape(exact.shape)
    want = sr.f16_sr(exact.astype(np.float32), sr.words(idx, seed))
    same = _bits_equal(ck, want)
    g64 = ck.astype(np.float64)
    spacing = np.maximum(sr.f16_grid(np.abs(exact))[1], sr.f16_grid(np.abs(g64))[1])
    slack = 1e-6 * np.abs(exact).max(axis=(-1, -2), keepdims=True)
    excess = np.abs(g64 - exact) - spacing - slack
    print(f"[gpu] f16 batch-256 flush: {same.mean():.6f} of sampled elements equal the oracle's "
          f"rounding; largest excess over one spacing {excess.max():.3g}", flush=True)
    assert (excess <= 0).all()
    assert same.mean() >= 0.999
    tok = work.steps
    yg = host(y)[:, sample, 0]
    args = (tok.x[:1][:, sample], tok.B[:1][:, sample], tok.C[:1][:, sample], tok.dt[:1][:, sample])
    _, y0 = orc_mod.conventional(exact, *args, work.A, work.D)
    _, yr = orc_mod.conventional(want, tok.x[:, sample], tok.B[:, sample], tok.C[:, sample],
                                 tok.dt[:, sample], work.A, work.D)
    assert_rows_close(yg[:1], y0, what="f16 batch-256 flushing call's outputs (sampled)")
    allow = np.stack([_spacing_allowance(want, tok.C[t][sample], shape.nheads) for t in range(1, steps)])
    assert_rows_close(yg[1:], yr[1:], what="f16 batch-256 non-flush outputs (sampled)", allowance=allow)
    assert np.all(host(st.meta)[:, :, 1] == steps)
    assert host(st.status)[0] == 0
