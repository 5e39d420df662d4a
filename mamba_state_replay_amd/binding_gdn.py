"""Python binding of the Gated DeltaNet entry points of libreplayssm.so
(include/replayssm_gdn.h; ctypes, argument marshalling only).

Same conventions as `binding`: torch device tensors, host-side checks of
device, dtype, shape and contiguity, no fallback (a missing library raises).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import binding as _rb
from .binding import _check, _expect, _ptr, _stream

GDN_NUM_BUFS = 5


class gdn_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "nv", "nk", "dk", "dv", "window", "max_drafts", "in_dtype", "ckpt_dtype")]


class gdn_state(ctypes.Structure):
    _fields_ = [("ckpt", ctypes.c_void_p), ("buf_k", ctypes.c_void_p), ("buf_u", ctypes.c_void_p),
                ("buf_g", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class gdn_tokens(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("T", ctypes.c_int32),
                ("sr_seed", ctypes.c_uint64)]


_P = ctypes.POINTER
_SIGS = {
    "gdn_row_blocks": (ctypes.c_int, [_P(gdn_config)]),
    "gdn_sizes": (ctypes.c_int, [_P(gdn_config), _P(ctypes.c_size_t)]),
    "gdn_decode_step": (ctypes.c_int, [_P(gdn_config), _P(gdn_state), _P(gdn_tokens), ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "gdn_verify_drafts": (ctypes.c_int, [_P(gdn_config), _P(gdn_state), _P(gdn_tokens), ctypes.c_void_p,
                                         ctypes.c_void_p]),
    "gdn_commit": (ctypes.c_int, [_P(gdn_config), _P(gdn_state), ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p]),
    "gdn_flush": (ctypes.c_int, [_P(gdn_config), _P(gdn_state), ctypes.c_uint64, ctypes.c_void_p]),
    "gdn_commit_verify": (ctypes.c_int, [_P(gdn_config), _P(gdn_state), ctypes.c_void_p, ctypes.c_int32,
                                         _P(gdn_tokens), ctypes.c_void_p, ctypes.c_void_p]),
    "gdn_conventional_update": (ctypes.c_int, [_P(gdn_config), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p, _P(gdn_tokens), ctypes.c_void_p, ctypes.c_void_p]),
    "gdn_conventional_commit": (ctypes.c_int, [_P(gdn_config), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
}
_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        handle = _rb.lib()
        for name, (res, args) in _SIGS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _LIB = handle
    return _LIB


@dataclass(frozen=True)
class GdnConfig:
    batch: int
    nv: int
    nk: int
    dk: int
    dv: int
    window: int = 16
    max_drafts: int = 1
    in_dtype: str = "bf16"
    ckpt_dtype: str = "f32"     # "f32", or "f16": FP16 checkpoint written with stochastic rounding

    @property
    def ckpt_torch(self) -> torch.dtype:
        return torch.float16 if self.ckpt_dtype == "f16" else torch.float32

    @property
    def cap(self) -> int:
        return self.window + 2 * self.max_drafts - 1

    @property
    def in_torch(self) -> torch.dtype:
        return torch.bfloat16 if self.in_dtype == "bf16" else torch.float32

    def c(self) -> gdn_config:
        return gdn_config(self.batch, self.nv, self.nk, self.dk, self.dv, self.window, self.max_drafts,
                          _rb.RSSM_BF16 if self.in_dtype == "bf16" else _rb.RSSM_F32,
                          _rb.RSSM_F16 if self.ckpt_dtype == "f16" else _rb.RSSM_F32)


def gdn_row_blocks(cfg: GdnConfig) -> int:
    c = cfg.c()
    return _check("gdn_row_blocks", lib().gdn_row_blocks(ctypes.byref(c)))


def gdn_sizes(cfg: GdnConfig) -> list[int]:
    c = cfg.c()
    out = (ctypes.c_size_t * GDN_NUM_BUFS)()
    _check("gdn_sizes", lib().gdn_sizes(ctypes.byref(c), out))
    return list(out)


@dataclass
class GdnState:
    ckpt: torch.Tensor      # [batch][nv][dv][dk] fp32 (fp16 with ckpt_dtype "f16")
    buf_k: torch.Tensor     # [batch][nk][cap][dk]
    buf_u: torch.Tensor     # [batch][nv][cap][dv] fp32
    buf_g: torch.Tensor     # [batch][nv][cap] fp32
    meta: torch.Tensor      # [batch][nv][row blocks][2] int32
    status: torch.Tensor | None

    @classmethod
    def allocate(cls, cfg: GdnConfig, device="cuda", status=True) -> "GdnState":
        sizes = gdn_sizes(cfg)
        b, nv, nk, dk, dv, cap = cfg.batch, cfg.nv, cfg.nk, cfg.dk, cfg.dv, cfg.cap
        parts = gdn_row_blocks(cfg)
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        st = cls(z((b, nv, dv, dk), cfg.ckpt_torch), z((b, nk, cap, dk), cfg.in_torch),
                 z((b, nv, cap, dv), torch.float32), z((b, nv, cap), torch.float32),
                 z((b, nv, parts, 2), torch.int32), z((1,), torch.int32) if status else None)
        for i, t in enumerate([st.ckpt, st.buf_k, st.buf_u, st.buf_g, st.meta]):
            assert t.numel() * t.element_size() == sizes[i], (i, sizes[i])
        return st

    def validate(self, cfg: GdnConfig):
        b, nv, nk, dk, dv, cap = cfg.batch, cfg.nv, cfg.nk, cfg.dk, cfg.dv, cfg.cap
        dev = self.ckpt.device
        _expect("ckpt", self.ckpt, (b, nv, dv, dk), cfg.ckpt_torch, dev)
        _expect("buf_k", self.buf_k, (b, nk, cap, dk), cfg.in_torch, dev)
        _expect("buf_u", self.buf_u, (b, nv, cap, dv), torch.float32, dev)
        _expect("buf_g", self.buf_g, (b, nv, cap), torch.float32, dev)
        _expect("meta", self.meta, (b, nv, gdn_row_blocks(cfg), 2), torch.int32, dev)
        if self.status is not None:
            _expect("status", self.status, (1,), torch.int32, dev)
        return dev

    def c(self) -> gdn_state:
        return gdn_state(*[_ptr(t) for t in (self.ckpt, self.buf_k, self.buf_u, self.buf_g, self.meta,
                                             self.status)])


@dataclass
class GdnTokens:
    """q, k [b][T][nk][dk]; v [b][T][nv][dv]; g, beta [b][T][nv] fp32."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    sr_seed: int = 0    # FP16 checkpoint: key of the call's stochastic rounding (vary it per call)

    @property
    def T(self) -> int:
        return self.q.shape[1]

    def validate(self, cfg: GdnConfig, device):
        b, T = cfg.batch, self.T
        _expect("q", self.q, (b, T, cfg.nk, cfg.dk), cfg.in_torch, device)
        _expect("k", self.k, (b, T, cfg.nk, cfg.dk), cfg.in_torch, device)
        _expect("v", self.v, (b, T, cfg.nv, cfg.dv), cfg.in_torch, device)
        _expect("g", self.g, (b, T, cfg.nv), torch.float32, device)
        _expect("beta", self.beta, (b, T, cfg.nv), torch.float32, device)

    def c(self) -> gdn_tokens:
        return gdn_tokens(_ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.g), _ptr(self.beta), self.T,
                          int(self.sr_seed) & 0xFFFFFFFFFFFFFFFF)


def _run(name, cfg, state, tokens, o, stream):
    dev = state.validate(cfg)
    tokens.validate(cfg, dev)
    _expect("o", o, (cfg.batch, tokens.T, cfg.nv, cfg.dv), torch.float32, dev)
    c, s, t = cfg.c(), state.c(), tokens.c()
    _check(name, getattr(lib(), name)(ctypes.byref(c), ctypes.byref(s), ctypes.byref(t), _ptr(o),
                                      _stream(stream)))


def gdn_decode_step(cfg: GdnConfig, state: GdnState, tokens: GdnTokens, o: torch.Tensor, stream=None):
    _run("gdn_decode_step", cfg, state, tokens, o, stream)


def gdn_verify_drafts(cfg: GdnConfig, state: GdnState, tokens: GdnTokens, o: torch.Tensor, stream=None):
    _run("gdn_verify_drafts", cfg, state, tokens, o, stream)


def gdn_commit_verify(cfg: GdnConfig, state: GdnState, accepted_prev: torch.Tensor, T_prev: int,
                      tokens: GdnTokens, o: torch.Tensor, stream=None):
    """gdn_commit(accepted_prev, T_prev) fused into this round's gdn_verify_drafts."""
    dev = state.validate(cfg)
    tokens.validate(cfg, dev)
    _expect("o", o, (cfg.batch, tokens.T, cfg.nv, cfg.dv), torch.float32, dev)
    _expect("accepted_prev", accepted_prev, (cfg.batch,), torch.int32, dev)
    c, s, t = cfg.c(), state.c(), tokens.c()
    _check("gdn_commit_verify", lib().gdn_commit_verify(ctypes.byref(c), ctypes.byref(s), _ptr(accepted_prev),
                                                        int(T_prev), ctypes.byref(t), _ptr(o), _stream(stream)))


def gdn_commit(cfg: GdnConfig, state: GdnState, accepted: torch.Tensor, T: int, stream=None):
    dev = state.validate(cfg)
    _expect("accepted", accepted, (cfg.batch,), torch.int32, dev)
    c, s = cfg.c(), state.c()
    _check("gdn_commit", lib().gdn_commit(ctypes.byref(c), ctypes.byref(s), _ptr(accepted), int(T),
                                          _stream(stream)))


def gdn_flush(cfg: GdnConfig, state: GdnState, sr_seed: int = 0, stream=None):
    state.validate(cfg)
    c, s = cfg.c(), state.c()
    _check("gdn_flush", lib().gdn_flush(ctypes.byref(c), ctypes.byref(s), int(sr_seed) & 0xFFFFFFFFFFFFFFFF,
                                        _stream(stream)))


def gdn_conventional_update(cfg: GdnConfig, states: torch.Tensor, tokens: GdnTokens, o: torch.Tensor,
                            nslots: int = 1, slot: torch.Tensor | None = None,
                            status: torch.Tensor | None = None, stream=None):
    """states: [batch][nv][dv][dk] (nslots 1, updated in place) or
    [batch][nslots][nv][dv][dk] with slot [batch] int32 (one snapshot per draft)."""
    dev = states.device
    shape = (cfg.batch, cfg.nv, cfg.dv, cfg.dk) if nslots == 1 else (cfg.batch, nslots, cfg.nv, cfg.dv, cfg.dk)
    _expect("states", states, shape, torch.float32, dev)
    tokens.validate(cfg, dev)
    _expect("o", o, (cfg.batch, tokens.T, cfg.nv, cfg.dv), torch.float32, dev)
    if nslots > 1:
        _expect("slot", slot, (cfg.batch,), torch.int32, dev)
    if status is not None:
        _expect("status", status, (1,), torch.int32, dev)
    c, t = cfg.c(), tokens.c()
    _check("gdn_conventional_update", lib().gdn_conventional_update(
        ctypes.byref(c), _ptr(states), int(nslots), _ptr(slot) if nslots > 1 else None, _ptr(status),
        ctypes.byref(t), _ptr(o), _stream(stream)))


def gdn_conventional_commit(cfg: GdnConfig, slot: torch.Tensor, nslots: int, accepted: torch.Tensor, T: int,
                            status: torch.Tensor | None = None, stream=None):
    dev = slot.device
    _expect("slot", slot, (cfg.batch,), torch.int32, dev)
    _expect("accepted", accepted, (cfg.batch,), torch.int32, dev)
    c = cfg.c()
    _check("gdn_conventional_commit", lib().gdn_conventional_commit(
        ctypes.byref(c), _ptr(slot), int(nslots), _ptr(accepted), int(T), _ptr(status), _stream(stream)))
