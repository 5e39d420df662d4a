"""Python binding of libreplayssm.so (ctypes; argument marshalling only).

The functions carry the C names of include/replayssm.h and take torch device
tensors.  Before any call the binding checks every tensor's device, dtype,
shape and contiguity against the config, because the C ABI receives bare
pointers.  Every computation runs in the library's HIP kernels; there is no
fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

import torch

PKG = Path(__file__).resolve().parent
LIBRARY = PKG / "libreplayssm.so"

RSSM_F32, RSSM_BF16, RSSM_FP8_E4M3, RSSM_NONE, RSSM_MXFP4, RSSM_MXFP8, RSSM_F16 = 0, 1, 2, 3, 4, 5, 6
RSSM_FLUSH_FORCE_CAST = 1
RSSM_STATUS_META, RSSM_STATUS_ACCEPT, RSSM_STATUS_SLOT = 1, 2, 4
RSSM_MAX_DRAFTS, RSSM_MAX_WINDOW = 8, 64
(BUF_CKPT, BUF_CKPT_READ, BUF_CKPT_SCALE, BUF_X, BUF_B, BUF_DT, BUF_META) = range(7)
NUM_BUFS = 7

_DTYPES = {"f32": RSSM_F32, "bf16": RSSM_BF16, "e4m3": RSSM_FP8_E4M3, None: RSSM_NONE,
           "none": RSSM_NONE, "mxfp4": RSSM_MXFP4, "mxfp8": RSSM_MXFP8, "f16": RSSM_F16}
_TORCH = {RSSM_F32: torch.float32, RSSM_BF16: torch.bfloat16, RSSM_FP8_E4M3: torch.uint8,
          RSSM_MXFP4: torch.uint8, RSSM_MXFP8: torch.uint8, RSSM_F16: torch.float16}


def _copy_shapes(rc, b, nh, hd, ds):
    """(ckpt_read shape, ckpt_scale shape and dtype) of a read-copy mode."""
    if rc == RSSM_MXFP4:
        return (b, nh, hd, ds // 2), ((b, nh, hd, ds // 32), torch.uint8)
    if rc == RSSM_MXFP8:
        return (b, nh, hd, ds), ((b, nh, hd, ds // 32), torch.uint8)
    if rc == RSSM_FP8_E4M3:
        return (b, nh, hd, ds), ((b, nh), torch.float32)
    return (b, nh, hd, ds), None


class rssm_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "nheads", "headdim", "dstate", "ngroups", "window", "max_drafts",
        "in_dtype", "read_copy", "ckpt_dtype")]


class rssm_state(ctypes.Structure):
    _fields_ = [("ckpt", ctypes.c_void_p), ("ckpt_read", ctypes.c_void_p),
                ("ckpt_scale", ctypes.c_void_p), ("buf_x", ctypes.c_void_p),
                ("buf_B", ctypes.c_void_p), ("buf_dt", ctypes.c_void_p),
                ("meta", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class rssm_tokens(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("dt", ctypes.c_void_p), ("T", ctypes.c_int32)]


class rssm_params(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("sr_seed", ctypes.c_uint64)]


_LIB = None

_SIGS = {
    "replayssm_capacity": (ctypes.c_int, [ctypes.POINTER(rssm_config)]),
    "replayssm_sizes": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.POINTER(ctypes.c_size_t)]),
    "replayssm_decode_step": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state),
                                             ctypes.POINTER(rssm_params), ctypes.POINTER(rssm_tokens),
                                             ctypes.c_void_p, ctypes.c_void_p]),
    "replayssm_flush": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state),
                                       ctypes.POINTER(rssm_params), ctypes.c_int32, ctypes.c_void_p]),
    "replayssm_verify_drafts": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state),
                                               ctypes.POINTER(rssm_params), ctypes.POINTER(rssm_tokens),
                                               ctypes.c_void_p, ctypes.c_void_p]),
    "replayssm_commit": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state),
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "replayssm_commit_verify": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state),
                                               ctypes.POINTER(rssm_params), ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.POINTER(rssm_tokens), ctypes.c_void_p,
                                               ctypes.c_void_p]),
    "conventional_state_update": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.c_void_p,
                                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.POINTER(rssm_params),
                                                 ctypes.POINTER(rssm_tokens), ctypes.c_void_p,
                                                 ctypes.c_void_p]),
    "conventional_commit": (ctypes.c_int, [ctypes.POINTER(rssm_config), ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "replayssm_last_error": (ctypes.c_char_p, []),
    "rssm_probe_sink_elems": (ctypes.c_size_t, [ctypes.c_size_t]),
    "rssm_probe_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "rssm_probe_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "rssm_probe_sr_f16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64,
                                         ctypes.c_uint64, ctypes.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not LIBRARY.exists():
            raise RuntimeError(f"{LIBRARY} is missing: build it with "
                               "`python -m mamba_state_replay_amd._build` (hipcc, gfx950)")
        handle = ctypes.CDLL(str(LIBRARY))
        for name, (res, args) in _SIGS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _LIB = handle
    return _LIB


class ReplaySSMError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().replayssm_last_error().decode(errors="replace")
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


def _check(fn, rc):
    if rc < 0:
        raise ReplaySSMError(fn, rc)
    return rc


@dataclass(frozen=True)
class Config:
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    window: int = 16
    max_drafts: int = 1
    in_dtype: str = "bf16"       # "f32" or "bf16"
    read_copy: str | None = None  # None, "bf16", "e4m3", "mxfp4" or "mxfp8"
    ckpt_dtype: str = "f32"       # "f32", or "f16": FP16 checkpoint written with stochastic rounding

    @property
    def cap(self) -> int:
        return self.window + 2 * self.max_drafts - 1

    @property
    def in_torch(self) -> torch.dtype:
        return _TORCH[_DTYPES[self.in_dtype]]

    def c(self) -> rssm_config:
        return rssm_config(self.batch, self.nheads, self.headdim, self.dstate, self.ngroups,
                           self.window, self.max_drafts, _DTYPES[self.in_dtype],
                           _DTYPES[self.read_copy], _DTYPES[self.ckpt_dtype])

    @property
    def ckpt_torch(self) -> torch.dtype:
        return _TORCH[_DTYPES[self.ckpt_dtype]]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(name, t, shape, dtype, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must live on the GPU ({device}), got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class State:
    """Device buffers of rssm_state (torch tensors, owned by the caller)."""
    ckpt: torch.Tensor
    ckpt_read: torch.Tensor | None
    ckpt_scale: torch.Tensor | None
    buf_x: torch.Tensor
    buf_B: torch.Tensor
    buf_dt: torch.Tensor
    meta: torch.Tensor          # [batch][nheads][2] {start, len}, one copy per head
    status: torch.Tensor | None

    @classmethod
    def allocate(cls, cfg: Config, device="cuda", status=True) -> "State":
        """Zeroed buffers with the shapes replayssm_sizes() reports."""
        sizes = replayssm_sizes(cfg)
        b, nh, hd, ds, ng, cap = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.cap
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        rc = _DTYPES[cfg.read_copy]
        read_shape, scale = _copy_shapes(rc, b, nh, hd, ds)
        st = cls(
            ckpt=z((b, nh, hd, ds), cfg.ckpt_torch),
            ckpt_read=None if rc == RSSM_NONE else z(read_shape, _TORCH[rc]),
            ckpt_scale=z(*scale) if scale else None,
            buf_x=z((b, nh, cap, hd), cfg.in_torch),
            buf_B=z((b, ng, cap, ds), cfg.in_torch),
            buf_dt=z((b, nh, cap), torch.float32),
            meta=z((b, nh, 2), torch.int32),
            status=z((1,), torch.int32) if status else None,
        )
        for i, t in enumerate([st.ckpt, st.ckpt_read, st.ckpt_scale, st.buf_x, st.buf_B, st.buf_dt,
                               st.meta]):
            nbytes = 0 if t is None else t.numel() * t.element_size()
            assert nbytes == sizes[i], (i, nbytes, sizes[i])
        return st

    def validate(self, cfg: Config):
        b, nh, hd, ds, ng, cap = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.cap
        dev = self.ckpt.device
        _expect("ckpt", self.ckpt, (b, nh, hd, ds), cfg.ckpt_torch, dev)
        rc = _DTYPES[cfg.read_copy]
        if rc == RSSM_NONE:
            if self.ckpt_read is not None or self.ckpt_scale is not None:
                raise ValueError("read_copy is None but ckpt_read/ckpt_scale are set")
        else:
            read_shape, scale = _copy_shapes(rc, b, nh, hd, ds)
            _expect("ckpt_read", self.ckpt_read, read_shape, _TORCH[rc], dev)
            if scale:
                _expect("ckpt_scale", self.ckpt_scale, scale[0], scale[1], dev)
            elif self.ckpt_scale is not None:
                raise ValueError("ckpt_scale is only used by the e4m3, mxfp4 and mxfp8 read copies")
        _expect("buf_x", self.buf_x, (b, nh, cap, hd), cfg.in_torch, dev)
        _expect("buf_B", self.buf_B, (b, ng, cap, ds), cfg.in_torch, dev)
        _expect("buf_dt", self.buf_dt, (b, nh, cap), torch.float32, dev)
        _expect("meta", self.meta, (b, nh, 2), torch.int32, dev)
        if self.status is not None:
            _expect("status", self.status, (1,), torch.int32, dev)
        return dev

    def c(self) -> rssm_state:
        return rssm_state(*[_ptr(t) for t in (self.ckpt, self.ckpt_read, self.ckpt_scale, self.buf_x,
                                              self.buf_B, self.buf_dt, self.meta, self.status)])


@dataclass
class Tokens:
    """T tokens per sequence: x [b][T][nh][hd], B/C [b][T][ng][ds], dt [b][T][nh]."""
    x: torch.Tensor
    B: torch.Tensor
    C: torch.Tensor
    dt: torch.Tensor

    @property
    def T(self) -> int:
        return self.x.shape[1]

    def validate(self, cfg: Config, device):
        b, nh, hd, ds, ng, T = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, self.T
        _expect("x", self.x, (b, T, nh, hd), cfg.in_torch, device)
        _expect("B", self.B, (b, T, ng, ds), cfg.in_torch, device)
        _expect("C", self.C, (b, T, ng, ds), cfg.in_torch, device)
        _expect("dt", self.dt, (b, T, nh), torch.float32, device)

    def c(self) -> rssm_tokens:
        return rssm_tokens(_ptr(self.x), _ptr(self.B), _ptr(self.C), _ptr(self.dt), self.T)


@dataclass
class Params:
    A: torch.Tensor
    D: torch.Tensor
    sr_seed: int = 0    # FP16 checkpoint: key of the call's stochastic rounding (vary it per call)

    def validate(self, cfg: Config, device):
        _expect("A", self.A, (cfg.nheads,), torch.float32, device)
        _expect("D", self.D, (cfg.nheads,), torch.float32, device)

    def c(self) -> rssm_params:
        return rssm_params(_ptr(self.A), _ptr(self.D), int(self.sr_seed) & 0xFFFFFFFFFFFFFFFF)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI).
# ---------------------------------------------------------------------------

def replayssm_capacity(cfg: Config) -> int:
    c = cfg.c()
    return _check("replayssm_capacity", lib().replayssm_capacity(ctypes.byref(c)))


def replayssm_sizes(cfg: Config) -> list[int]:
    c = cfg.c()
    out = (ctypes.c_size_t * NUM_BUFS)()
    _check("replayssm_sizes", lib().replayssm_sizes(ctypes.byref(c), out))
    return list(out)


def replayssm_decode_step(cfg: Config, state: State, params: Params, tokens: Tokens,
                          y: torch.Tensor, stream=None) -> None:
    dev = state.validate(cfg)
    params.validate(cfg, dev)
    tokens.validate(cfg, dev)
    _expect("y", y, (cfg.batch, tokens.T, cfg.nheads, cfg.headdim), torch.float32, dev)
    c, s, p, t = cfg.c(), state.c(), params.c(), tokens.c()
    _check("replayssm_decode_step", lib().replayssm_decode_step(
        ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), ctypes.byref(t), _ptr(y), _stream(stream)))


def replayssm_flush(cfg: Config, state: State, params: Params, flags: int = 0, stream=None) -> None:
    dev = state.validate(cfg)
    params.validate(cfg, dev)
    c, s, p = cfg.c(), state.c(), params.c()
    _check("replayssm_flush", lib().replayssm_flush(
        ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), int(flags), _stream(stream)))


def replayssm_verify_drafts(cfg: Config, state: State, params: Params, tokens: Tokens,
                            y: torch.Tensor, stream=None) -> None:
    dev = state.validate(cfg)
    params.validate(cfg, dev)
    tokens.validate(cfg, dev)
    _expect("y", y, (cfg.batch, tokens.T, cfg.nheads, cfg.headdim), torch.float32, dev)
    c, s, p, t = cfg.c(), state.c(), params.c(), tokens.c()
    _check("replayssm_verify_drafts", lib().replayssm_verify_drafts(
        ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), ctypes.byref(t), _ptr(y), _stream(stream)))


def replayssm_commit(cfg: Config, state: State, accepted: torch.Tensor, T: int, stream=None) -> None:
    dev = state.validate(cfg)
    _expect("accepted", accepted, (cfg.batch,), torch.int32, dev)
    c, s = cfg.c(), state.c()
    _check("replayssm_commit", lib().replayssm_commit(
        ctypes.byref(c), ctypes.byref(s), _ptr(accepted), int(T), _stream(stream)))


def replayssm_commit_verify(cfg: Config, state: State, params: Params, accepted_prev: torch.Tensor,
                            T_prev: int, tokens: Tokens, y: torch.Tensor, stream=None) -> None:
    dev = state.validate(cfg)
    params.validate(cfg, dev)
    tokens.validate(cfg, dev)
    _expect("accepted_prev", accepted_prev, (cfg.batch,), torch.int32, dev)
    _expect("y", y, (cfg.batch, tokens.T, cfg.nheads, cfg.headdim), torch.float32, dev)
    c, s, p, t = cfg.c(), state.c(), params.c(), tokens.c()
    _check("replayssm_commit_verify", lib().replayssm_commit_verify(
        ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), _ptr(accepted_prev), int(T_prev),
        ctypes.byref(t), _ptr(y), _stream(stream)))


def conventional_state_update(cfg: Config, states: torch.Tensor, params: Params, tokens: Tokens,
                              y: torch.Tensor, slot: torch.Tensor | None = None,
                              status: torch.Tensor | None = None, stream=None) -> None:
    """states: [batch][nslots][nheads][headdim][dstate] fp32 (nslots = states.shape[1])."""
    if states.dim() != 5:
        raise ValueError("states must be [batch][nslots][nheads][headdim][dstate]")
    dev = states.device
    nslots = states.shape[1]
    _expect("states", states, (cfg.batch, nslots, cfg.nheads, cfg.headdim, cfg.dstate),
            torch.float32, dev)
    params.validate(cfg, dev)
    tokens.validate(cfg, dev)
    if nslots > 1:
        _expect("slot", slot, (cfg.batch,), torch.int32, dev)
    if status is not None:
        _expect("status", status, (1,), torch.int32, dev)
    _expect("y", y, (cfg.batch, tokens.T, cfg.nheads, cfg.headdim), torch.float32, dev)
    c, p, t = cfg.c(), params.c(), tokens.c()
    _check("conventional_state_update", lib().conventional_state_update(
        ctypes.byref(c), _ptr(states), nslots, _ptr(slot) if nslots > 1 else None, _ptr(status),
        ctypes.byref(p), ctypes.byref(t), _ptr(y), _stream(stream)))


def conventional_commit(cfg: Config, slot: torch.Tensor, nslots: int, accepted: torch.Tensor, T: int,
                        status: torch.Tensor | None = None, stream=None) -> None:
    dev = slot.device
    _expect("slot", slot, (cfg.batch,), torch.int32, dev)
    _expect("accepted", accepted, (cfg.batch,), torch.int32, dev)
    if status is not None:
        _expect("status", status, (1,), torch.int32, dev)
    c = cfg.c()
    _check("conventional_commit", lib().conventional_commit(
        ctypes.byref(c), _ptr(slot), int(nslots), _ptr(accepted), int(T), _ptr(status), _stream(stream)))


def replayssm_last_error() -> str:
    return lib().replayssm_last_error().decode(errors="replace")


def rssm_probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    need = lib().rssm_probe_sink_elems(nbytes)
    _expect("sink", sink, (need,), torch.float32, src.device)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _check("rssm_probe_read", lib().rssm_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


def rssm_probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("dst and src must be contiguous and the same size")
    _check("rssm_probe_copy", lib().rssm_probe_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def rssm_probe_sr_f16(src: torch.Tensor, dst: torch.Tensor, vec0: int, seed: int, stream=None) -> None:
    """dst (fp16) = the FP16 checkpoint flush's stochastic rounding of src (fp32),
    value i with the random word of checkpoint vector vec0 + i // 4."""
    if src.dtype != torch.float32 or dst.dtype != torch.float16 or src.numel() != dst.numel():
        raise ValueError("src fp32 and dst fp16 of the same size")
    if not (src.is_contiguous() and dst.is_contiguous()) or src.device.type != "cuda":
        raise ValueError("contiguous GPU tensors required")
    _check("rssm_probe_sr_f16", lib().rssm_probe_sr_f16(_ptr(src), _ptr(dst), src.numel(), int(vec0), int(seed),
                                                        _stream(stream)))


def probe_sink_elems(nbytes: int) -> int:
    return int(lib().rssm_probe_sink_elems(nbytes))
