"""Exhaustive checks of the read-copy casts on the GPU.

The casts run inside the flush kernel (replayssm_flush with FORCE_CAST on a
state with no records: the FP32 checkpoint is only read and cast).  Expected
codes come from the host encoders of tests/formats.py, written from the format
definitions and pinned against torch on the CPU:

* bf16: every one of the 2^32 fp32 bit patterns, round to nearest even, NaN
  stays NaN; the FP32 checkpoint is left bit-for-bit unchanged;
* e4m3fn: every fp32 pattern with |v| <= 448, in tiles whose largest magnitude
  is 448 so the per-tile scale is exactly 1 and the code is the encoding of v
  itself; NaN inputs give a NaN code.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from mamba_state_replay_amd import binding as rb
from tests import formats
from tests.gpu_util import device, host, say

pytestmark = pytest.mark.gpu

TILE = 64 * 128


def _encode(fn, x, dtype, sub=2 ** 18, workers=8):
    """fn over x in cache-sized slices on a few threads (numpy releases the GIL)."""
    out = np.empty(x.size, dtype)

    def job(i):
        out[i:i + sub] = fn(x[i:i + sub])
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(job, range(0, x.size, sub)))
    return out


def _cast_state(copy, batch, dev):
    cfg = rb.Config(batch, 128, 64, 128, 8, window=16, max_drafts=1, in_dtype="bf16", read_copy=copy)
    st = rb.State.allocate(cfg, dev)        # no records: a FORCE_CAST flush only casts
    p = rb.Params(torch.full((128,), -1.0, device=dev), torch.zeros(128, device=dev))
    return cfg, st, p


def test_bf16_cast_every_fp32_pattern():
    dev = device()
    batch = 512                              # 2^29 patterns per launch, 8 launches
    per = batch * 128 * TILE
    cfg, st, p = _cast_state("bf16", batch, dev)
    bad = 0
    for c in range(2 ** 32 // per):
        say(f"bf16 cast, patterns {c * per:#x} ..")
        bits = np.arange(c * per, (c + 1) * per, dtype=np.uint64).astype(np.uint32)
        src = torch.from_numpy(bits.view(np.int32)).to(dev)
        st.ckpt.view(torch.int32).view(-1).copy_(src)
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
        torch.cuda.synchronize()
        assert torch.equal(st.ckpt.view(torch.int32).view(-1), src), "cast-only flush wrote the FP32 checkpoint"
        got = host(st.ckpt_read.view(torch.int16)).view(np.uint16).ravel()
        want = _encode(formats.encode_bf16_bits, bits, np.uint16)
        gn, wn = formats.bf16_is_nan(got), formats.bf16_is_nan(want)
        mism = (gn != wn) | (~wn & (got != want))
        if mism.any():
            i = np.flatnonzero(mism)[:5]
            print(f"[gpu] mismatches at fp32 patterns {bits[i]} -> got {got[i]} want {want[i]}", flush=True)
        bad += int(mism.sum())
        del src
    assert bad == 0, f"{bad} fp32 patterns cast to the wrong bf16"


def test_e4m3_cast_every_pattern_up_to_448():
    dev = device()
    top = int(np.float32(448.0).view(np.uint32))          # 0x43E00000
    mags = np.arange(0, top + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | np.uint32(0x80000000)])
    per_tile = TILE - 1                                     # element 0 of each tile holds 448
    ntiles = -(-pats.size // per_tile)
    batch = 256
    tiles_per_launch = batch * 128
    cfg, st, p = _cast_state("e4m3", batch, dev)
    anchor = np.float32(448.0).view(np.uint32)
    bad = 0
    for t0 in range(0, ntiles, tiles_per_launch):
        say(f"e4m3 cast, tiles {t0} .. of {ntiles}")
        nt = min(tiles_per_launch, ntiles - t0)
        chunk = pats[t0 * per_tile:(t0 + nt) * per_tile]
        tiles = np.zeros((tiles_per_launch, TILE), np.uint32)
        flat = tiles[:nt, 1:].reshape(-1)
        flat[:chunk.size] = chunk
        tiles[:nt, 1:] = flat.reshape(nt, per_tile)
        tiles[:, 0] = anchor
        st.ckpt.view(torch.int32).view(-1).copy_(torch.from_numpy(tiles.view(np.int32).reshape(-1)))
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
        torch.cuda.synchronize()
        assert np.all(host(st.ckpt_scale) == 1.0), "per-tile scale of a tile with absmax 448 must be 1"
        got = host(st.ckpt_read).reshape(tiles_per_launch, TILE)[:nt, 1:].reshape(-1)[:chunk.size]
        want = _encode(formats.encode_e4m3fn_fast, chunk.view(np.float32), np.uint8)
        mism = ~formats.same_code(got, want)
        if mism.any():
            i = np.flatnonzero(mism)[:5]
            print(f"[gpu] mismatches at fp32 patterns {chunk[i]} -> got {got[i]} want {want[i]}", flush=True)
        bad += int(mism.sum())
    assert bad == 0, f"{bad} fp32 values cast to the wrong e4m3 code"


def test_e4m3_cast_of_nan_is_nan():
    """A NaN in the FP32 state must stay visible in the e4m3 copy (code 0x7F or
    0xFF), not turn into a finite value; the tile's other values keep scale 1."""
    dev = device()
    cfg, st, p = _cast_state("e4m3", 1, dev)
    g = np.random.default_rng(9)
    vals = g.uniform(-448, 448, size=(128, TILE)).astype(np.float32)
    vals[:, 0] = 448.0
    nan_bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF, 0xFFFFFFFF], np.uint32)
    pos = g.integers(1, TILE, size=(128, nan_bits.size))
    for h in range(128):
        vals[h, pos[h]] = nan_bits.view(np.float32)
    st.ckpt.copy_(torch.from_numpy(vals.reshape(1, 128, 64, 128)))
    say("e4m3 cast of NaN")
    rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
    torch.cuda.synchronize()
    got = host(st.ckpt_read).reshape(128, TILE)
    isnan = np.isnan(vals)
    assert np.all((got[isnan] & 0x7F) == 0x7F), f"NaN inputs gave codes {np.unique(got[isnan])}"
    assert np.all(formats.same_code(got[~isnan], formats.encode_e4m3fn(vals[~isnan])))
    assert np.all(host(st.ckpt_scale) == 1.0)


def _mx_cast_every_pattern(copy, top, anchor, scale_byte, want_fn):
    """Every fp32 pattern with magnitude up to the pattern top, 31 to a block
    of 32 whose first lane holds anchor (the block's largest magnitude, which
    fixes its scale byte): the codes against want_fn(values)."""
    dev = device()
    mags = np.arange(0, top + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | np.uint32(0x80000000)])
    per_blk = 31
    nblk = -(-pats.size // per_blk)
    batch = 256
    blocks_per_launch = batch * 128 * TILE // 32
    cfg = rb.Config(batch, 128, 64, 128, 8, window=16, max_drafts=1, in_dtype="bf16", read_copy=copy)
    st = rb.State.allocate(cfg, dev)
    p = rb.Params(torch.full((128,), -1.0, device=dev), torch.zeros(128, device=dev))
    bad = 0
    for b0 in range(0, nblk, blocks_per_launch):
        say(f"{copy} cast, blocks {b0} .. of {nblk}")
        nb = min(blocks_per_launch, nblk - b0)
        chunk = pats[b0 * per_blk:(b0 + nb) * per_blk]
        blk = np.zeros((blocks_per_launch, 32), np.uint32)
        flat = blk[:nb, 1:].reshape(-1)
        flat[:chunk.size] = chunk
        blk[:nb, 1:] = flat.reshape(nb, per_blk)
        blk[:, 0] = np.float32(anchor).view(np.uint32)
        st.ckpt.view(torch.int32).view(-1).copy_(torch.from_numpy(blk.view(np.int32).reshape(-1)))
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
        torch.cuda.synchronize()
        assert np.all(host(st.ckpt_scale) == scale_byte), f"every block's scale byte is {scale_byte}"
        if copy == "mxfp4":
            packed = host(st.ckpt_read).reshape(blocks_per_launch, 16)
            codes = np.empty((blocks_per_launch, 32), np.uint8)
            codes[:, 0::2] = packed & 0xF
            codes[:, 1::2] = packed >> 4
            zero_mask = 7
        else:
            codes = host(st.ckpt_read).reshape(blocks_per_launch, 32)
            zero_mask = 0x7F
        got = codes[:nb, 1:].reshape(-1)[:chunk.size]
        want = want_fn(chunk.view(np.float32))
        mism = (got != want) & ~(((got & zero_mask) == 0) & ((want & zero_mask) == 0))
        if mism.any():
            i = np.flatnonzero(mism)[:5]
            print(f"[gpu] mismatches at fp32 patterns {chunk[i]} -> got {got[i]} want {want[i]}", flush=True)
        bad += int(mism.sum())
    assert bad == 0, f"{bad} fp32 values cast to the wrong {copy} code"


def test_mxfp4_cast_every_pattern_below_8():
    """Every fp32 value with |v| < 8, in MXFP4 blocks whose largest magnitude
    lies in [4, 8) (one lane of each block holds 4.0), so the block scale is
    2^0 and each code is the E2M1 encoding of v itself (nearest, ties to even,
    saturating at 6)."""
    top = int(np.nextafter(np.float32(8.0), np.float32(0)).view(np.uint32))
    _mx_cast_every_pattern("mxfp4", top, 4.0, 127,
                           lambda v: _encode(formats.e2m1_encode_fast, v, np.uint8))


def test_mxfp8_cast_every_pattern_up_to_448():
    """Every fp32 value with |v| <= 448, in MXFP8 blocks whose largest magnitude
    is 448 (one lane of each block holds it), so the block scale is 2^0 and
    each code is the e4m3 encoding of v itself (nearest, ties to even)."""
    top = int(np.float32(448.0).view(np.uint32))
    _mx_cast_every_pattern("mxfp8", top, 448.0, 127,
                           lambda v: _encode(formats.encode_e4m3fn_fast, v, np.uint8))
