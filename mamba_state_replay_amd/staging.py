"""Host -> device staging of seeded workloads into the library's layouts.

Pure data movement: token arrays drawn as [steps][batch][...] become device
tensors in the [batch][T][...] layout of rssm_tokens, and a workload's
pre-committed records are copied into ring slots 0..n0[b]-1 with meta =
{0, n0[b]}.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as rb
from . import synth


def _dev(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def _in_array(tokens: synth.Tokens, name: str):
    """Storage array of x/B/C and the torch dtype it is viewed as."""
    if tokens.in_dtype == "bf16":
        return getattr(tokens, name + "_bits").view(np.int16), torch.bfloat16
    return getattr(tokens, name).astype(np.float32), None


def tokens_block(tokens: synth.Tokens, t0: int, t1: int, device) -> rb.Tokens:
    """Tokens t0..t1-1 as one call's rssm_tokens ([batch][T][...])."""
    out = {}
    for name in ("x", "B", "C"):
        arr, dt = _in_array(tokens, name)
        out[name] = _dev(np.swapaxes(arr[t0:t1], 0, 1), device, dt)
    out["dt"] = _dev(np.swapaxes(tokens.dt[t0:t1].astype(np.float32), 0, 1), device)
    return rb.Tokens(**out)


class TokenStream:
    """Every token of a run resident on the device; step(t) is a T=1 view."""

    def __init__(self, tokens: synth.Tokens, device, T: int = 1):
        if tokens.steps % T:
            raise ValueError("steps must be a multiple of T")
        self.T = T
        self.calls = tokens.steps // T
        self._t = {}
        for name in ("x", "B", "C"):
            arr, dt = _in_array(tokens, name)
            # [calls][T][batch][...] -> [calls][batch][T][...]
            shp = (self.calls, T) + arr.shape[1:]
            self._t[name] = _dev(np.swapaxes(arr.reshape(shp), 1, 2), device, dt)
        dts = tokens.dt.astype(np.float32).reshape((self.calls, T) + tokens.dt.shape[1:])
        self._t["dt"] = _dev(np.swapaxes(dts, 1, 2), device)

    def call(self, i: int) -> rb.Tokens:
        return rb.Tokens(self._t["x"][i], self._t["B"][i], self._t["C"][i], self._t["dt"][i])

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self._t.values())


def params(work: synth.Workload, device) -> rb.Params:
    return rb.Params(_dev(work.A.astype(np.float32), device), _dev(work.D.astype(np.float32), device))


def config(shape: synth.LayerShape, in_dtype="bf16", read_copy=None, window=None,
           max_drafts=None, ckpt_dtype="f32") -> rb.Config:
    return rb.Config(shape.batch, shape.nheads, shape.headdim, shape.dstate, shape.ngroups,
                     window if window is not None else shape.window,
                     max_drafts if max_drafts is not None else shape.max_drafts,
                     in_dtype, read_copy, ckpt_dtype)


def replay_state(cfg: rb.Config, work: synth.Workload, device) -> rb.State:
    """State with ckpt = h0 and the n0[b] pre-committed records in slots 0..n0[b]-1
    (ring pointer {0, n0[b]} in every head's copy).  An FP16 checkpoint holds h0
    rounded to the nearest fp16."""
    if int(work.n0.max(initial=0)) > cfg.cap:
        raise ValueError("pre-committed records exceed the ring capacity")
    st = rb.State.allocate(cfg, device)
    st.ckpt.copy_(torch.from_numpy(work.h0.astype(np.float32)).to(st.ckpt.dtype))
    npre = work.pre.steps
    if npre:
        b, nh, hd, ds, ng, cap = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.cap
        keep = (np.arange(npre)[None, :] < work.n0[:, None])           # [batch][npre]
        xs, xdt = _in_array(work.pre, "x")
        Bs, _ = _in_array(work.pre, "B")
        bx = np.zeros((b, nh, cap, hd), xs.dtype)
        bB = np.zeros((b, ng, cap, ds), Bs.dtype)
        bdt = np.zeros((b, nh, cap), np.float32)
        bx[:, :, :npre] = np.transpose(xs, (1, 2, 0, 3)) * keep[:, None, :, None]
        bB[:, :, :npre] = np.transpose(Bs, (1, 2, 0, 3)) * keep[:, None, :, None]
        bdt[:, :, :npre] = np.transpose(work.pre.dt.astype(np.float32), (1, 2, 0)) * keep[:, None, :]
        st.buf_x.copy_(_dev(bx, "cpu", xdt))
        st.buf_B.copy_(_dev(bB, "cpu", xdt))
        st.buf_dt.copy_(torch.from_numpy(bdt))
    meta = np.stack([np.zeros_like(work.n0), work.n0], axis=1).astype(np.int32)   # [batch][2]
    st.meta.copy_(torch.from_numpy(np.repeat(meta[:, None, :], cfg.nheads, axis=1)))
    return st


def conventional_states(cfg: rb.Config, h: np.ndarray, nslots: int, device) -> torch.Tensor:
    """[batch][nslots][nheads][headdim][dstate] with slot 0 = h."""
    st = torch.zeros((cfg.batch, nslots, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32,
                     device=device)
    st[:, 0].copy_(torch.from_numpy(np.asarray(h, np.float32)))
    return st


class GdnTokenStream:
    """Every GDN token of a run resident on the device, as [calls][batch][T][...];
    call(i) is the i-th call's gdn_tokens (pure data movement)."""

    def __init__(self, tokens, device, T: int = 1):
        from . import binding_gdn as bg
        self._bg = bg
        if tokens.steps % T:
            raise ValueError("steps must be a multiple of T")
        self.T = T
        self.calls = tokens.steps // T
        self._t = {}
        for name in ("q", "k", "v", "g", "beta"):
            arr = tokens.storage(name)
            dt = None
            if arr.dtype == np.uint16:
                arr, dt = arr.view(np.int16), torch.bfloat16
            else:
                arr = arr.astype(np.float32)
            shp = (self.calls, T) + arr.shape[1:]
            self._t[name] = _dev(np.swapaxes(arr.reshape(shp), 1, 2), device, dt)

    def call(self, i: int):
        return self._bg.GdnTokens(*(self._t[n][i] for n in ("q", "k", "v", "g", "beta")))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self._t.values())
