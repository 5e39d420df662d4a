"""GPU tests of the dual-precision mode: FP32 checkpoint + a bf16, e4m3 (one
scale per tile), MXFP4 or MXFP8 (an E8M0 scale per 32 columns) read copy.

* the kernels' e4m3 decoding of every finite code, and their encodings on the
  cast-only and the flush paths, against host encoders written from the format
  definitions (tests/formats.py);
* outputs read from the copy stay within the stated bound of the fp64 oracle;
* the copy never enters the recurrence: the FP32 checkpoint is bit-identical
  to an FP32-only run, and a NaN-poisoned copy leaves every flush unchanged
  (blog section "Benefit 3: Limit error accumulation with separate
  precisions").
"""
import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from mamba_state_replay_amd import staging, synth
from oracle import oracle as orc_mod
from tests import formats
from tests.gpu_util import TOL, assert_rows_close, device, head_err, host, say

pytestmark = pytest.mark.gpu

NEMO = dict(nheads=128, headdim=64, dstate=128, ngroups=8)
SHAPES = {
    "16x16": dict(nheads=4, headdim=16, dstate=16, ngroups=1),
    "64x64": dict(nheads=16, headdim=64, dstate=64, ngroups=2),
    "64x128": NEMO,
    "128x128": dict(nheads=8, headdim=128, dstate=128, ngroups=1),
}
UNIT = {"bf16": 2.0 ** -8, "e4m3": 2.0 ** -4, "mxfp4": 2.0 ** -2, "mxfp8": 2.0 ** -4}   # relative bound of one read
MX = ("mxfp4", "mxfp8")


def read_delta(copy, scale, hd, ds):
    """Absolute part of the per-element read bound, broadcastable to
    [batch][nheads][hd][ds]: 0 for bf16; half the e4m3 subnormal step, s 2^-10,
    for e4m3 (one scale s per tile); a quarter of the block scale X, half the
    E2M1 spacing below 1, for MXFP4, and X 2^-10, half the e4m3 subnormal step,
    for MXFP8 (scales [batch][nheads][hd][ds / 32] E8M0).
    A margin of 1e-3 covers fp32 rounding."""
    if copy == "bf16":
        return 0.0
    scale = np.asarray(scale)
    if copy == "e4m3":
        return (scale.astype(np.float64) * 2.0 ** -10 * 1.001)[..., None, None]
    if copy == "mxfp8":
        return np.repeat(formats.e8m0_value(scale) * 2.0 ** -10 * 1.001, 32, axis=-1)
    return np.repeat(formats.e8m0_value(scale) / 4 * 1.001, 32, axis=-1)


def test_e4m3_decode_every_code():
    """Tile (16 x 16) holding all 256 codes (NaN codes replaced by 0), scale 1,
    x = 0, dt = 0, C = unit vectors: each output is exactly one decoded code."""
    dev = device()
    T = 8
    cfg = rb.Config(1, 4, 16, 16, 1, window=4, max_drafts=T, in_dtype="f32", read_copy="e4m3")
    st = rb.State.allocate(cfg, dev)
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    st.ckpt_read[0, 0].copy_(torch.from_numpy(codes.reshape(16, 16)))
    st.ckpt_scale.fill_(1.0)
    p = rb.Params(torch.full((4,), -1.0, device=dev), torch.zeros(4, device=dev))
    got = np.zeros((16, 16))
    say("e4m3 decode of every code")
    for j0 in (0, 8):
        C = torch.zeros((1, T, 1, 16), device=dev)
        for q in range(T):
            C[0, q, 0, j0 + q] = 1.0
        tok = rb.Tokens(torch.zeros((1, T, 4, 16), device=dev), torch.zeros((1, T, 1, 16), device=dev),
                        C, torch.zeros((1, T, 4), device=dev))
        y = torch.empty((1, T, 4, 16), device=dev)
        rb.replayssm_verify_drafts(cfg, st, p, tok, y)
        torch.cuda.synchronize()
        got[:, j0:j0 + T] = host(y)[0, :, 0, :].T
    expect = formats.decode_e4m3fn(codes).reshape(16, 16)
    assert np.array_equal(got, expect)


def _crafted_values(g, n):
    """Every finite e4m3 value, every tie between neighbours, values next to the
    ties, and random magnitudes over the whole range, all within +-448."""
    val, nan = formats.e4m3fn_table()
    fin = np.unique(val[~nan])
    mids = (fin[1:] + fin[:-1]) / 2
    pool = np.concatenate([fin, mids, np.nextafter(mids, -1e9), np.nextafter(mids, 1e9),
                           np.exp(g.uniform(-16, 6, n)) * g.choice([-1.0, 1.0], n)])
    pool = np.clip(pool, -448, 448).astype(np.float32)
    return g.choice(pool, n)


@pytest.mark.parametrize("copy", ["bf16", "e4m3"])
def test_cast_only_encoding(copy):
    """flush(FORCE_CAST) with nothing to fold: copy = encode(checkpoint)."""
    dev = device()
    g = np.random.default_rng(21)
    cfg = rb.Config(2, 8, 64, 128, 8, window=16, max_drafts=1, in_dtype="bf16", read_copy=copy)
    st = rb.State.allocate(cfg, dev)
    h = _crafted_values(g, 2 * 8 * 64 * 128).reshape(2, 8, 64, 128)
    h[:, :, 0, 0] = 448.0          # absmax 448 in every tile: e4m3 scale is exactly 1
    h[:, :, 0, 1] = -448.0
    st.ckpt.copy_(torch.from_numpy(h))
    p = rb.Params(torch.full((8,), -1.0, device=dev), torch.zeros(8, device=dev))
    say(f"cast-only flush {copy}")
    rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
    torch.cuda.synchronize()
    assert torch.equal(st.ckpt.cpu(), torch.from_numpy(h)), "cast-only flush changed the FP32 checkpoint"
    if copy == "bf16":
        ref = torch.from_numpy(h).to(torch.bfloat16)
        assert torch.equal(st.ckpt_read.cpu().view(torch.int16), ref.view(torch.int16))
    else:
        assert np.all(host(st.ckpt_scale) == 1.0)
        got = host(st.ckpt_read)
        assert np.all(formats.same_code(got, formats.encode_e4m3fn(h)))


def unpack_fp4(packed):
    """[..., ds / 2] bytes -> [..., ds] E2M1 codes (low nibble = even column)."""
    b = np.asarray(packed, np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def same_fp4(got_scales, got_codes, want_scales, want_codes):
    """Equal scales, and equal codes where the block is not NaN (+0 and -0 one value)."""
    if not np.array_equal(got_scales, want_scales):
        return False
    live = np.repeat(want_scales != 255, 32, axis=-1)
    same = (got_codes == want_codes) | (((got_codes & 7) == 0) & ((want_codes & 7) == 0))
    return bool(np.all(same | ~live))


def same_fp8(got_scales, got_codes, want_scales, want_codes):
    """Equal scales, and equal e4m3 codes (+0 and -0 one value, any NaN code
    equal to any other)."""
    if not np.array_equal(got_scales, want_scales):
        return False
    both_nan = ((np.asarray(got_codes) & 0x7F) == 0x7F) & ((np.asarray(want_codes) & 0x7F) == 0x7F)
    return bool(np.all(formats.same_code(got_codes, want_codes) | both_nan))


def same_mx(copy, st, want):
    """The state's MX copy equals the host encoding want = (scales, codes)."""
    if copy == "mxfp4":
        return same_fp4(host(st.ckpt_scale), unpack_fp4(host(st.ckpt_read)), *want)
    return same_fp8(host(st.ckpt_scale), host(st.ckpt_read), *want)


def mx_encode(copy, h):
    return formats.mxfp4_encode(h) if copy == "mxfp4" else formats.mxfp8_encode(h)


@pytest.mark.parametrize("copy", MX)
def test_mx_cast_only_encoding(copy):
    """flush(FORCE_CAST) with nothing to fold writes the MX encoding of the
    checkpoint: blocks over 40 orders of magnitude, a grid of code values and
    midpoints (every E2M1 value and midpoint; the top binades of e4m3) times
    the block scale, blocks whose largest magnitude sits at the edge of the
    scale rule, zero blocks, a block with a NaN, and fp32 subnormals; codes and
    E8M0 scales against the host encoder."""
    dev = device()
    g = np.random.default_rng(22)
    cfg = rb.Config(2, 8, 64, 128, 8, window=16, max_drafts=1, in_dtype="bf16", read_copy=copy)
    st = rb.State.allocate(cfg, dev)
    h = (np.exp(g.uniform(-45, 45, (2, 8, 64, 4, 1))) * g.standard_normal((2, 8, 64, 4, 32))).astype(np.float32)
    if copy == "mxfp4":
        grid = np.concatenate([formats.E2M1, (formats.E2M1[1:] + formats.E2M1[:-1]) / 2])      # 15 values
        top = 6.0
    else:   # e4m3 values and midpoints from 240 to 448, and a subnormal midpoint
        grid = np.concatenate([np.arange(240.0, 449.0, 16.0), [1.5 * 2.0 ** -9]])       # 15 values
        top = 448.0
    h[0, 0, :, 0, :15] = grid * 2.0 ** g.integers(-20, 20, (64, 1))
    h[0, 0, :, 0, 15] = top * 2.0 ** g.integers(-20, 20, 64)
    # largest magnitude just above / at / below a power-of-two multiple of the top code
    edge = (top * 2.0 ** g.integers(-20, 20, (64, 1))).astype(np.float32)
    h[0, 4, :, 1:, :] = (edge[:, :, None] * g.uniform(-0.9, 0.9, (64, 3, 32))).astype(np.float32)
    h[0, 4, :, 1, 0] = np.nextafter(edge[:, 0], np.float32(np.inf))
    h[0, 4, :, 2, 0] = edge[:, 0]
    h[0, 4, :, 3, 0] = np.nextafter(edge[:, 0], np.float32(0))
    h[0, 1, :, 1, :] = 0.0
    h[0, 2, 5, 2, 7] = np.nan
    h[1, 3, :, 3, :] = np.float32(1e-41) * g.standard_normal((64, 32)).astype(np.float32)
    h = h.reshape(2, 8, 64, 128)
    st.ckpt.copy_(torch.from_numpy(h))
    p = rb.Params(torch.full((8,), -1.0, device=dev), torch.zeros(8, device=dev))
    say(f"cast-only flush {copy}")
    rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
    torch.cuda.synchronize()
    assert torch.equal(st.ckpt.cpu().view(torch.int32), torch.from_numpy(h).view(torch.int32)), \
        "cast-only flush changed the FP32 checkpoint"
    assert same_mx(copy, st, mx_encode(copy, h))


def test_block_scales_keep_small_rows():
    """Rows of one tile whose magnitudes span 2^-24 .. 1 (outlier channels):
    with one e4m3 scale per tile the smallest rows fall below the e4m3 range
    and read back as zero, while the MXFP8 copy (a scale per 32 columns) keeps
    every row's largest read error within 2^-4 of the row's largest magnitude
    (its per-element bound |v| 2^-4 + X 2^-10, X <= that magnitude / 224)."""
    dev = device()
    g = np.random.default_rng(23)
    h = g.standard_normal((2, 8, 64, 128)).astype(np.float32)
    h *= (2.0 ** -g.uniform(0, 24, (2, 8, 64, 1))).astype(np.float32)
    h[:, :, 0, 0] = 4.0                                   # every tile keeps a large row
    p = rb.Params(torch.full((8,), -1.0, device=dev), torch.zeros(8, device=dev))
    row_err = {}
    for copy in ("e4m3", "mxfp8"):
        cfg = rb.Config(2, 8, 64, 128, 8, window=16, max_drafts=1, in_dtype="bf16", read_copy=copy)
        st = rb.State.allocate(cfg, dev)
        st.ckpt.copy_(torch.from_numpy(h))
        say(f"row magnitudes, cast-only flush {copy}")
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
        torch.cuda.synchronize()
        codes = host(st.ckpt_read)
        if copy == "e4m3":
            dec = formats.decode_e4m3fn(codes) * host(st.ckpt_scale)[:, :, None, None]
        else:
            dec = formats.mxfp8_decode(host(st.ckpt_scale), codes)
        row_err[copy] = np.abs(dec - h).max(axis=-1) / np.abs(h).max(axis=-1)
    small = np.abs(h).max(axis=-1) < 2.0 ** -17         # under half e4m3's smallest step at scale 4/448
    print(f"[gpu] row magnitudes: worst row read error e4m3 {row_err['e4m3'].max():.3g} "
          f"({int(small.sum())} rows read as zero), mxfp8 {row_err['mxfp8'].max():.3g}", flush=True)
    assert small.sum() > 100 and np.all(row_err["e4m3"][small] == 1.0)
    assert row_err["mxfp8"].max() <= 2.0 ** -4 * 1.001


@pytest.mark.parametrize("copy", ["bf16", "e4m3", "mxfp4", "mxfp8"])
def test_flush_encoding_and_scale(copy):
    """A real flush (5 committed records): the copy is the encoding of the new
    FP32 checkpoint, with scale absmax/448 per tile for e4m3."""
    dev = device()
    shape = synth.LayerShape(batch=3, window=16, **NEMO)
    work = synth.decode_workload(shape, 0, seed=1010, n0=5)
    cfg = staging.config(shape, read_copy=copy)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    say(f"flush encoding {copy}")
    rb.replayssm_flush(cfg, st, p)
    torch.cuda.synchronize()
    H = host(st.ckpt)
    assert np.all(host(st.meta)[:, :, 1] == 0)
    if copy == "bf16":
        ref = torch.from_numpy(H).to(torch.bfloat16)
        assert torch.equal(st.ckpt_read.cpu().view(torch.int16), ref.view(torch.int16))
    elif copy in MX:
        assert same_mx(copy, st, mx_encode(copy, H.astype(np.float32)))
    else:
        amax = np.abs(H).max(axis=(-1, -2)).astype(np.float32)
        sc = (amax / np.float32(448.0)).astype(np.float32)
        assert np.array_equal(host(st.ckpt_scale), sc)
        inv = (np.float32(1.0) / sc).astype(np.float32)
        x = (H * inv[:, :, None, None]).astype(np.float32)
        assert np.all(formats.same_code(host(st.ckpt_read), formats.encode_e4m3fn(x)))


def _run_dual(cfg, work, dev, steps, poison_before=()):
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev)
    if cfg.read_copy:
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
    y = torch.empty((steps, cfg.batch, 1, cfg.nheads, cfg.headdim), device=dev)
    scales = {}
    for t in range(steps):
        if t in poison_before:
            if cfg.read_copy == "bf16":
                st.ckpt_read.view(torch.int16).fill_(0x7FC0)
            elif cfg.read_copy == "e4m3":
                st.ckpt_read.fill_(0x7F)
            elif cfg.read_copy == "mxfp4":
                st.ckpt_read.fill_(0xFF)          # E2M1 -6 in both nibbles, block scales NaN
                st.ckpt_scale.fill_(255)
            else:
                st.ckpt_read.fill_(0x7F)          # e4m3 NaN, block scales NaN
                st.ckpt_scale.fill_(255)
        rb.replayssm_decode_step(cfg, st, p, stream.call(t), y[t])
        if cfg.read_copy in ("e4m3",) + MX:
            scales[t] = st.ckpt_scale.clone()
    torch.cuda.synchronize()
    return host(y)[:, :, 0], st, {k: host(v) for k, v in scales.items()}


@pytest.mark.parametrize("tile", ["64x128", "16x16", "64x64", "128x128"])
@pytest.mark.parametrize("copy", ["bf16", "e4m3", "mxfp4", "mxfp8"])
def test_dual_precision_error_bound(copy, tile):
    """Outputs of non-flush steps read the copy; per element
    |y - y_ref| <= d_q sum_j |C_q[j]| (u |H_s[i,j]| + delta) + 1e-4 * (head output scale),
    u = 2^-8 (bf16), 2^-4 (e4m3, MXFP8) or 2^-2 (MXFP4), delta = 0 (bf16), s 2^-10
    (e4m3, half the subnormal step scaled), X / 4 (MXFP4, X the block's scale) or
    X 2^-10 (MXFP8),
    H_s the oracle state at the last flush, d_q the decay since then.  Flushing
    steps read FP32 registers and meet the FP32 tolerance.  The FP32 checkpoint
    must be bit-identical to an FP32-only run."""
    if copy in MX and SHAPES[tile]["dstate"] % 32:
        pytest.skip("MX blocks are 32 columns of dstate")
    dev = device()
    L, steps = 16, 72
    shape = synth.LayerShape(batch=4, window=L, **SHAPES[tile])
    work = synth.decode_workload(shape, steps, seed=1011, n0=L)
    say(f"dual precision {copy} {tile}, 72 steps")
    cfg32 = staging.config(shape)
    y32, st32, _ = _run_dual(cfg32, work, dev, steps)
    cfgc = staging.config(shape, read_copy=copy)
    yc, stc, scales = _run_dual(cfgc, work, dev, steps)
    assert torch.equal(st32.ckpt, stc.ckpt), "read copy changed the FP32 recurrence"
    assert torch.equal(st32.meta, stc.meta)

    yref, _ = orc_mod.decode(work, nsteps=steps)
    # the explicit FORCE_CAST flush folds the L pre-filled records; then a
    # flush happens at the start of steps L, 2L, ...
    flush_steps = set(range(L, steps, L))
    hs = {}
    for tf in [0] + sorted(flush_steps):
        _, hs[tf] = orc_mod.decode(work, nsteps=tf)
    scale = np.abs(yref).max(axis=(0, 3))      # per (seq, head) output scale
    worst_ratio, per_window = 0.0, []
    for tf in sorted(hs):
        win = [t for t in range(tf, min(tf + L, steps)) if t not in flush_steps]
        Hs = hs[tf]
        werr = 0.0
        for t in win:
            dec = np.exp(work.A[None, :] * work.steps.dt[tf:t + 1].astype(np.float64).sum(0))  # [b][h]
            Cg = np.repeat(work.steps.C[t].astype(np.float64), shape.nheads // shape.ngroups, axis=1)  # [b][h][ds]
            sc = scales[max(x for x in [0] + sorted(flush_steps) if x <= t)] if copy != "bf16" else None
            delta = read_delta(copy, sc, shape.headdim, shape.dstate)
            term = UNIT[copy] * np.abs(Hs) + delta                      # [b][h][hd][ds]
            bound = dec[:, :, None] * np.einsum("bhij,bhj->bhi", term, np.abs(Cg)) + 1e-4 * scale[:, :, None]
            err = np.abs(yc[t] - yref[t])
            worst_ratio = max(worst_ratio, float((err / bound).max()))
            werr = max(werr, float((err / scale[:, :, None]).max()))
        per_window.append(werr)
    print(f"[gpu] {copy}: worst error/bound {worst_ratio:.3f}; max normalized error per window {per_window}")
    assert worst_ratio <= 1.0
    # read error does not grow with length: every window's error is of the same size as the first's
    assert max(per_window) <= 4 * per_window[0] + 1e-4
    fl = sorted(flush_steps)
    assert_rows_close(yc[fl], yref[fl], what=f"{copy} flushing-step outputs")


@pytest.mark.parametrize("copy", ["bf16", "e4m3", "mxfp4", "mxfp8"])
def test_poisoned_copy_never_enters_recurrence(copy):
    """NaN-fill the copy right before a flushing step: that step's outputs (read
    from FP32 registers) and the checkpoint it writes are unchanged, and later
    steps read the freshly written copy."""
    dev = device()
    L, steps = 8, 20
    shape = synth.LayerShape(batch=3, window=L, **NEMO)
    work = synth.decode_workload(shape, steps, seed=1012, n0=L)
    cfg = staging.config(shape, read_copy=copy)
    say(f"poisoned {copy} copy")
    y_clean, st_clean, _ = _run_dual(cfg, work, dev, steps)
    y_pois, st_pois, _ = _run_dual(cfg, work, dev, steps, poison_before=(L, 2 * L))
    assert np.all(np.isfinite(y_pois))
    assert np.array_equal(y_clean, y_pois)
    assert torch.equal(st_clean.ckpt, st_pois.ckpt)
    assert torch.equal(st_clean.ckpt_read, st_pois.ckpt_read)
    if copy != "bf16":
        assert torch.equal(st_clean.ckpt_scale, st_pois.ckpt_scale)


def test_dual_4096_steps_bound_and_no_drift():
    """4096 decode steps, 8 sequences x 128 heads, L = 16, all five modes run
    side by side, window by window, against the fp64 oracle stepped over the
    same window:
    * FP32-only outputs within the FP32 tolerance in every window;
    * read-copy outputs within the per-element bound of the dual-precision
      test above in every window (flushing steps read FP32 registers and meet
      the FP32 tolerance);
    * the copy never enters the recurrence: after 4096 steps the FP32
      checkpoints of the five modes are bit-identical;
    * the read error does not grow: the largest normalized error of the last
      quarter of windows is no more than twice that of the first quarter."""
    dev = device()
    L, steps = 16, 4096
    shape = synth.LayerShape(batch=8, window=L, **NEMO)
    work = synth.decode_workload(shape, steps, seed=1005, n0=L)
    modes = (None, "bf16", "e4m3", "mxfp4", "mxfp8")
    cfgs = {m: staging.config(shape, read_copy=m) for m in modes}
    sts = {m: staging.replay_state(cfgs[m], work, dev) for m in modes}
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev)
    say("dual precision, 4096 steps, 8 sequences, five modes")
    for m in modes[1:]:
        rb.replayssm_flush(cfgs[m], sts[m], p, rb.RSSM_FLUSH_FORCE_CAST)
    rb.replayssm_flush(cfgs[None], sts[None], p)
    H = orc_mod.committed_state(work)                 # H_s of window 0
    A = work.A.astype(np.float64)
    hpg = shape.nheads // shape.ngroups
    y = {m: torch.empty((L, 8, 1, 128, 64), device=dev) for m in modes}
    per_window = {m: [] for m in modes}
    worst_ratio = {m: 0.0 for m in modes[1:]}
    for w in range(steps // L):
        t0 = w * L
        scales = {}
        for t in range(t0, t0 + L):
            for m in modes:
                rb.replayssm_decode_step(cfgs[m], sts[m], p, stream.call(t), y[m][t - t0])
            if t == t0:
                scales = {m: host(sts[m].ckpt_scale) for m in ("e4m3",) + MX}
        torch.cuda.synchronize()
        tok = work.steps
        Hs = H
        H, yref = orc_mod.default().conventional(Hs, tok.x[t0:t0 + L], tok.B[t0:t0 + L], tok.C[t0:t0 + L],
                                                 tok.dt[t0:t0 + L], work.A, work.D)
        scale = np.abs(yref).max(axis=(0, 3))                       # per (seq, head)
        # steps of this window that read the copy (step t0 flushes, except in window 0)
        copy_rows = np.arange(L) if w == 0 else np.arange(1, L)
        dsum = np.cumsum(tok.dt[t0:t0 + L].astype(np.float64), axis=0)      # [L][b][h]
        dec = np.exp(A[None, None, :] * dsum)                        # decay since H_s, [L][b][h]
        Cabs = torch.from_numpy(np.repeat(np.abs(tok.C[t0:t0 + L].astype(np.float64)), hpg, axis=2))  # [L][b][h][ds]
        Habs = torch.from_numpy(np.abs(Hs))                           # [b][h][hd][ds]
        HC = torch.einsum("bhij,tbhj->tbhi", Habs, Cabs).numpy()     # [L][b][h][hd]
        Csum = Cabs.sum(-1).numpy()                                   # [L][b][h]
        for m in modes:
            got = host(y[m])[:, :, 0].astype(np.float64)
            err = np.abs(got - yref)
            if m is None:
                per_window[m].append(float((err.max(axis=(0, 3)) / scale).max()))
                assert per_window[m][-1] <= TOL, f"fp32 window {w}: {per_window[m][-1]:.3e}"
                continue
            per_window[m].append(float((err[copy_rows].max(axis=(0, 3)) / scale).max()))
            read = UNIT[m] * HC                                       # u sum_j |H_s[i,j]| |C_q[j]|
            if m == "e4m3":
                read = read + (scales[m] * 2.0 ** -10 * 1.001)[None, :, :, None] * Csum[..., None]
            elif m in MX:                                       # sum_j |C_q[j]| delta(i, j)
                Xq = torch.from_numpy(np.ascontiguousarray(read_delta(m, scales[m], 64, 128)))
                read = read + torch.einsum("bhij,tbhj->tbhi", Xq, Cabs).numpy()
            bound = dec[..., None] * read + TOL * scale[None, :, :, None]
            ratio = float((err[copy_rows] / bound[copy_rows]).max())
            worst_ratio[m] = max(worst_ratio[m], ratio)
            assert ratio <= 1.0, f"{m} window {w}: error / bound {ratio:.3f}"
            if w > 0:
                fl = float((err[0].max(axis=-1) / scale).max())
                assert fl <= TOL, f"{m} flushing step of window {w}: {fl:.3e}"
    for m in modes[1:]:
        assert torch.equal(sts[m].ckpt, sts[None].ckpt), f"{m}: read copy changed the FP32 recurrence"
    q = len(per_window[None]) // 4
    for m in modes:
        pw = np.array(per_window[m])
        print(f"[gpu] {m or 'fp32'}: max error per window first quarter {pw[:q].max():.3e}, "
              f"last quarter {pw[-q:].max():.3e}, mean {pw.mean():.3e}"
              + (f", worst error/bound {worst_ratio[m]:.3f}" if m else ""), flush=True)
        if m:
            assert pw[-q:].max() <= 2 * pw[:q].max(), f"{m}: read error grows over the run"


COPY_VERIFY_SHAPES = {
    "64x128": NEMO,                                                    # 4 (e4m3) / 2 (bf16) heads per workgroup
    "64x64": SHAPES["64x64"],
    "hpg2": dict(nheads=6, headdim=64, dstate=128, ngroups=3),         # 2 heads per group
    "hpg1": dict(nheads=5, headdim=64, dstate=128, ngroups=5),         # one head per group
}


@pytest.mark.parametrize("T", [3, 8])
@pytest.mark.parametrize("tile", list(COPY_VERIFY_SHAPES))
@pytest.mark.parametrize("copy", ["bf16", "e4m3", "mxfp4", "mxfp8"])
def test_copy_verify_rounds(copy, tile, T):
    """Speculative rounds (verify + commit) with a read copy beside the same
    rounds in FP32-only mode: the FP32 checkpoint and ring pointers of the two
    runs stay bit-identical (the copy never enters the recurrence).  Against
    the fp64 oracle's verification rounds: outputs of rounds that flush
    (computed from fresh FP32 registers) meet the FP32 tolerance; in the other
    rounds the error is the copy's read error plus the FP32 one and must lie
    within d_q sum_j |C_q[j]| (u |H_s[i,j]| + delta) + 1e-4 of the head's
    output scale per element (u and delta as in the dual-precision bound,
    delta from the copy's scales), with H_s the oracle's state at the
    sequence's last flush and d_q the decay since then."""
    _copy_verify(copy, tile, T, L=8, rounds=14)


@pytest.mark.parametrize("copy", ["e4m3", "mxfp4", "mxfp8"])
def test_copy_verify_long_window(copy):
    """The same check at L = 16 with T = 8 drafts on the benchmarked layer:
    windows of up to 23 rows, so the staging list of the 4-head copy
    workgroups (x rows of four heads, the group's B rows, the drafts' C rows,
    the MX scale bytes) outgrows the vectors each thread issues up front and
    the rest goes through the staging loop."""
    n_max = _copy_verify(copy, "64x128", 8, L=16, rounds=12)
    # a round with 11 committed records stages 4 x 19 x 8 + 19 x 16 + 8 x 16 + 64 = 1104 vectors
    assert n_max >= 11, f"no round reached 11 committed records (max {n_max})"


def _copy_verify(copy, tile, T, L, rounds):
    dev = device()
    shape = synth.LayerShape(batch=2, window=L, max_drafts=T, **COPY_VERIFY_SHAPES[tile])
    work = synth.verify_workload(shape, rounds, T, seed=1015)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    p = staging.params(work, dev)
    stream = staging.TokenStream(work.steps, dev, T=T)
    say(f"copy verify {copy} {tile} T={T} L={L}")
    runs = {}
    for mode in (None, copy):
        cfg = staging.config(shape, read_copy=mode)
        st = staging.replay_state(cfg, work, dev)
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST if mode else 0)
        ys, hs, scs, metas = [], [], [], []
        y = torch.empty((shape.batch, T, shape.nheads, shape.headdim), device=dev)
        for r in range(rounds):
            rb.replayssm_verify_drafts(cfg, st, p, stream.call(r), y)
            rb.replayssm_commit(cfg, st, acc[r], T)
            ys.append(host(y).copy())
            hs.append(host(st.ckpt).astype(np.float64))
            metas.append(host(st.meta).copy())
            if mode in ("e4m3",) + MX:
                scs.append(host(st.ckpt_scale).copy())
        torch.cuda.synchronize()
        assert int(host(st.status)[0]) == 0
        runs[mode] = (ys, hs, scs, metas)
    y32, h32, _, m32 = runs[None]
    yc, hc, scc, mc = runs[copy]
    yref, _ = orc_mod.verify_rounds(work)                  # [rounds][T][batch][nheads][headdim]
    # the oracle's state after the commits of the first r rounds: H_s of a flush at the start of round r
    Hr = [orc_mod.verify_rounds(work, rounds=r)[1] for r in range(rounds)]
    A = work.A.astype(np.float64)
    hpg = shape.nheads // shape.ngroups
    dt = work.steps.dt.astype(np.float64)                  # [rounds * T][batch][nheads]
    C = work.steps.C.astype(np.float64)                    # [rounds * T][batch][ngroups][dstate]
    n = np.zeros(shape.batch, np.int64)                    # committed records since the last flush
    seg = np.zeros((shape.batch, shape.nheads))            # sum of their dt
    last = np.zeros(shape.batch, np.int64)                 # round of the last flush (0: the explicit one)
    worst = 0.0
    n_max = 0                                              # most committed records a non-flushing round found
    for r in range(rounds):
        assert np.array_equal(hc[r], h32[r]), f"round {r}: read copy changed the FP32 checkpoint"
        assert np.array_equal(mc[r], m32[r])
        flushed = n >= L
        n_max = max(n_max, int(np.where(flushed, 0, n).max()))
        n = np.where(flushed, 0, n)
        seg = np.where(flushed[:, None], 0.0, seg)
        last = np.where(flushed, r, last)
        scale = np.abs(yref[r]).max(axis=(0, 3))           # per (seq, head)
        for b in range(shape.batch):
            d_run = seg[b].copy()
            for q in range(T):
                t = r * T + q
                d_run = d_run + dt[t, b]
                diff = np.abs(yc[r][b, q].astype(np.float64) - yref[r][q, b])    # [h][hd]
                if flushed[b]:
                    assert float((diff.max(axis=-1) / scale[b]).max()) <= TOL, f"round {r} seq {b}: flush outputs"
                    continue
                Cq = np.repeat(np.abs(C[t, b]), hpg, axis=0)                     # [h][ds]
                Hs = np.abs(Hr[last[b]][b])                                      # [h][hd][ds]
                read = UNIT[copy] * np.einsum("hij,hj->hi", Hs, Cq)
                if copy == "e4m3":
                    read = read + (scc[r][b] * 2.0 ** -10 * 1.001)[:, None] * Cq.sum(-1)[:, None]
                elif copy in MX:
                    read = read + np.einsum("hij,hj->hi", read_delta(copy, scc[r][b], 0, 0), Cq)
                bound = np.exp(A * d_run)[:, None] * read * 1.001 + TOL * scale[b][:, None]
                ratio = float((diff / bound).max())
                worst = max(worst, ratio)
                assert ratio <= 1.0, f"round {r} seq {b} draft {q}: error / bound {ratio:.3f}"
        a_r = work.extra["accepted"][r]
        for b in range(shape.batch):
            seg[b] += dt[r * T:r * T + a_r[b], b].sum(axis=0)
        n = n + a_r
    print(f"[gpu] {copy} {tile} T={T} L={L}: worst error/bound {worst:.3f}, most committed records {n_max}",
          flush=True)
    return n_max


@pytest.mark.parametrize("copy", ["bf16", "e4m3", "mxfp4", "mxfp8"])
def test_dual_full_batch_sampled(copy):
    """The benchmarked layer (batch 256, L = 16) with each read copy, 40 steps
    (flushes at the starts of steps 16 and 32): the FP32 checkpoint and the
    ring pointers are bit-identical to an FP32-only run over the whole batch;
    on sampled sequences the non-flush outputs stay within the read bound of
    test_dual_precision_error_bound and the flushing steps meet the FP32
    tolerance."""
    dev = device()
    L, steps = 16, 40
    shape = synth.NEMOTRON3
    work = synth.decode_workload(shape, steps, seed=1012, n0=L)
    say(f"dual precision {copy}, batch 256, {steps} steps")
    _, st32, _ = _run_dual(staging.config(shape), work, dev, steps)
    yc, stc, scales = _run_dual(staging.config(shape, read_copy=copy), work, dev, steps)
    assert torch.equal(st32.ckpt, stc.ckpt), "read copy changed the FP32 recurrence"
    assert torch.equal(st32.meta, stc.meta)
    del st32
    seqs = np.array([0, 77, 128, 255])
    yc = yc[:, seqs]
    yref, _ = orc_mod.decode(work, nsteps=steps, seqs=seqs)
    flush_steps = [16, 32]
    scale = np.abs(yref).max(axis=(0, 3))
    worst = 0.0
    for tf in [0] + flush_steps:
        _, Hs = orc_mod.decode(work, nsteps=tf, seqs=seqs)
        for t in range(tf, min(tf + L, steps)):
            if t in flush_steps:
                continue
            dec = np.exp(work.A[None, :] * work.steps.dt[tf:t + 1][:, seqs].astype(np.float64).sum(0))
            Cg = np.repeat(work.steps.C[t][seqs].astype(np.float64), shape.nheads // shape.ngroups, axis=1)
            sc = scales[max(x for x in [0] + flush_steps if x <= t)][seqs] if copy != "bf16" else None
            term = UNIT[copy] * np.abs(Hs) + read_delta(copy, sc, shape.headdim, shape.dstate)
            bound = dec[:, :, None] * np.einsum("bhij,bhj->bhi", term, np.abs(Cg)) + 1e-4 * scale[:, :, None]
            worst = max(worst, float((np.abs(yc[t] - yref[t]) / bound).max()))
    print(f"[gpu] {copy} batch 256: worst error/bound {worst:.3f}", flush=True)
    assert worst <= 1.0
    assert_rows_close(yc[flush_steps], yref[flush_steps], what=f"{copy} batch-256 flushing-step outputs")
    assert host(stc.status)[0] == 0
