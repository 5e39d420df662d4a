"""The C-ABI library loads and exports every function include/*.h declares;
host-side checks reject bad arguments before anything reaches the GPU."""
import ctypes
import re
import subprocess
import sys
from pathlib import Path

import pytest
import torch

ROOT = Path(__file__).resolve().parent.parent
HEADERS = sorted((ROOT / "include").glob("*.h"))


@pytest.fixture(scope="module")
def rb():
    from mamba_state_replay_amd import binding
    if not binding.LIBRARY.exists():
        from mamba_state_replay_amd import _build
        _build.build()
    binding.lib()
    return binding


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith(("#", "typedef", "return")):
                names.add(m.group(1))
    return sorted(names)


def test_headers_declare_the_entry_points():
    names = declared_functions()
    for required in ["replayssm_decode_step", "replayssm_flush", "replayssm_verify_drafts",
                     "replayssm_commit", "conventional_state_update", "conventional_commit",
                     "replayssm_sizes", "replayssm_capacity", "replayssm_last_error"]:
        assert required in names, required


def test_library_exports_every_declared_symbol(rb):
    out = subprocess.run(["nm", "-D", "--defined-only", str(rb.LIBRARY)], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    handle = ctypes.CDLL(str(rb.LIBRARY))
    for n in declared_functions():
        getattr(handle, n)


def test_sizes_and_capacity(rb):
    cfg = rb.Config(batch=256, nheads=128, headdim=64, dstate=128, ngroups=8, window=16, max_drafts=1)
    assert rb.replayssm_capacity(cfg) == 17
    sz = rb.replayssm_sizes(cfg)
    assert sz[rb.BUF_CKPT] == 256 * 128 * 64 * 128 * 4 == 1 << 30   # 4 MiB per sequence
    assert sz[rb.BUF_CKPT_READ] == 0 and sz[rb.BUF_CKPT_SCALE] == 0
    assert sz[rb.BUF_X] == 256 * 128 * 17 * 64 * 2
    assert sz[rb.BUF_B] == 256 * 8 * 17 * 128 * 2
    assert sz[rb.BUF_DT] == 256 * 128 * 17 * 4
    assert sz[rb.BUF_META] == 256 * 128 * 8 and len(sz) == 7
    e4 = rb.Config(256, 128, 64, 128, 8, 16, 3, "bf16", "e4m3")
    assert rb.replayssm_capacity(e4) == 21
    sz = rb.replayssm_sizes(e4)
    assert sz[rb.BUF_CKPT_READ] == 1 << 28 and sz[rb.BUF_CKPT_SCALE] == 256 * 128 * 4
    # MX copies: one E8M0 byte per 32 columns; E2M1 codes two to a byte, e4m3 one
    for mode, code_bytes in (("mxfp4", 1 << 27), ("mxfp8", 1 << 28)):
        sz = rb.replayssm_sizes(rb.Config(256, 128, 64, 128, 8, 16, 1, "bf16", mode))
        assert sz[rb.BUF_CKPT_READ] == code_bytes and sz[rb.BUF_CKPT_SCALE] == 256 * 128 * 64 * 128 // 32


def test_f16_checkpoint_sizes_and_combinations(rb):
    """An FP16 checkpoint takes 2 bytes per element; it is read directly or
    through an MXFP4 copy, and the conventional state stays fp32."""
    sz = rb.replayssm_sizes(rb.Config(256, 128, 64, 128, 8, 16, 1, "bf16", None, "f16"))
    assert sz[rb.BUF_CKPT] == 256 * 128 * 64 * 128 * 2 and sz[rb.BUF_CKPT_READ] == 0
    sz = rb.replayssm_sizes(rb.Config(256, 128, 64, 128, 8, 16, 1, "bf16", "mxfp4", "f16"))
    assert sz[rb.BUF_CKPT] == 256 * 128 * 64 * 128 * 2 and sz[rb.BUF_CKPT_SCALE] == 256 * 128 * 64 * 128 // 32
    for copy in ("bf16", "e4m3", "mxfp8"):
        with pytest.raises(rb.ReplaySSMError) as e:
            rb.replayssm_sizes(rb.Config(4, 128, 64, 128, 8, 16, 1, "bf16", copy, "f16"))
        assert e.value.code == -3
    L = rb.lib()
    c = rb.Config(4, 128, 64, 128, 8, ckpt_dtype="f16").c()
    p = rb.rssm_params()
    t = rb.rssm_tokens(None, None, None, None, 1)
    assert L.conventional_state_update(ctypes.byref(c), None, 1, None, None, ctypes.byref(p),
                                       ctypes.byref(t), None, None) == -3
    bad = rb.Config(4, 128, 64, 128, 8).c()
    bad.ckpt_dtype = 1                                   # bf16 is no checkpoint type
    assert L.replayssm_sizes(ctypes.byref(bad), (ctypes.c_size_t * 8)()) == -3


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_mx_copies_need_blocks_of_32_columns(rb, mode):
    with pytest.raises(rb.ReplaySSMError) as e:
        rb.replayssm_sizes(rb.Config(4, 4, 16, 16, 1, 4, 1, "f32", mode))
    assert e.value.code == -2 and "32" in str(e.value)
    rb.replayssm_sizes(rb.Config(4, 16, 64, 64, 2, 4, 1, "f32", mode))     # dstate 64: accepted


@pytest.mark.parametrize("bad,code", [
    (dict(headdim=32), -2), (dict(ngroups=3), -2), (dict(window=0), -2), (dict(window=65), -2),
    (dict(max_drafts=9), -2), (dict(max_drafts=0), -2), (dict(batch=-1), -2),
])
def test_config_rejections(rb, bad, code):
    base = dict(batch=4, nheads=128, headdim=64, dstate=128, ngroups=8, window=16, max_drafts=1)
    base.update(bad)
    with pytest.raises(rb.ReplaySSMError) as e:
        rb.replayssm_sizes(rb.Config(**base))
    assert e.value.code == code


def test_null_pointers_rejected_before_launch(rb):
    L = rb.lib()
    c = rb.Config(4, 128, 64, 128, 8).c()
    s = rb.rssm_state()          # all NULL
    p = rb.rssm_params()
    t = rb.rssm_tokens(None, None, None, None, 1)
    assert L.replayssm_decode_step(ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), ctypes.byref(t),
                                   None, None) == -1
    assert "required" in rb.replayssm_last_error()
    assert L.replayssm_flush(ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), 0, None) == -1
    assert L.replayssm_flush(ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), 8, None) == -2
    assert L.replayssm_commit(ctypes.byref(c), ctypes.byref(s), None, 2, None) == -4
    assert L.replayssm_commit(ctypes.byref(c), ctypes.byref(s), None, 1, None) == -1
    assert L.conventional_state_update(ctypes.byref(c), None, 1, None, None, ctypes.byref(p),
                                       ctypes.byref(t), None, None) == -1
    assert L.conventional_commit(ctypes.byref(c), None, 1, None, 1, None, None) == -2
    assert L.replayssm_decode_step(None, None, None, None, None, None) == -1
    assert L.replayssm_commit_verify(ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), None, 1,
                                     ctypes.byref(t), None, None) == -1
    assert L.replayssm_commit_verify(ctypes.byref(c), ctypes.byref(s), ctypes.byref(p), None, 0,
                                     ctypes.byref(t), None, None) == -4
    bad = rb.Config(4, 128, 64, 128, 8, in_dtype="bf16").c()
    bad.in_dtype = 7
    assert L.replayssm_sizes(ctypes.byref(bad), (ctypes.c_size_t * 8)()) == -3


def test_binding_checks_tensors_on_host(rb):
    cfg = rb.Config(2, 8, 16, 16, 2, window=4, max_drafts=1, in_dtype="f32")
    # CPU tensors are refused before the library is called
    st = rb.State(*[torch.zeros(1)] * 8)
    p = rb.Params(torch.zeros(8), torch.zeros(8))
    tok = rb.Tokens(torch.zeros(2, 1, 8, 16), torch.zeros(2, 1, 2, 16), torch.zeros(2, 1, 2, 16),
                    torch.zeros(2, 1, 8))
    with pytest.raises(ValueError):
        rb.replayssm_decode_step(cfg, st, p, tok, torch.zeros(2, 1, 8, 16))


def test_gdn_sizes_and_rejections(rb):
    from mamba_state_replay_amd import binding_gdn as bg
    cfg = bg.GdnConfig(batch=512, nv=32, nk=16, dk=128, dv=128, window=16, max_drafts=1)
    assert bg.gdn_row_blocks(cfg) == 2
    sz = bg.gdn_sizes(cfg)
    assert sz[0] == 512 * 32 * 128 * 128 * 4 == 1 << 30          # 2 MiB per sequence
    assert sz[1] == 512 * 16 * 17 * 128 * 2                      # bf16 keys
    assert sz[2] == 512 * 32 * 17 * 128 * 4                      # fp32 corrected values
    assert sz[3] == 512 * 32 * 17 * 4 and sz[4] == 512 * 32 * 2 * 2 * 4
    assert bg.gdn_row_blocks(bg.GdnConfig(2, 4, 2, 16, 32, 4)) == 2
    for bad in [dict(dk=64), dict(dv=96), dict(nk=3), dict(nv=0), dict(window=0), dict(window=65),
                dict(max_drafts=9), dict(batch=-1)]:
        base = dict(batch=4, nv=32, nk=16, dk=128, dv=128, window=16, max_drafts=1)
        base.update(bad)
        with pytest.raises(rb.ReplaySSMError) as e:
            bg.gdn_sizes(bg.GdnConfig(**base))
        assert e.value.code == -2, bad
    c = bg.GdnConfig(4, 32, 16, 128, 128).c()
    c.in_dtype = 7
    assert bg.lib().gdn_sizes(ctypes.byref(c), (ctypes.c_size_t * 5)()) == -3
    c = bg.GdnConfig(4, 32, 16, 128, 128).c()
    c.ckpt_dtype = 2
    assert bg.lib().gdn_sizes(ctypes.byref(c), (ctypes.c_size_t * 5)()) == -3
    assert bg.gdn_sizes(bg.GdnConfig(512, 32, 16, 128, 128, ckpt_dtype="f16"))[0] == 1 << 29
    # LDS bound: dk = 128 takes window 40 at 8 drafts and window 64 at 4, not window 48 or 64 at 8
    bg.gdn_sizes(bg.GdnConfig(2, 32, 16, 128, 128, 40, 8))
    bg.gdn_sizes(bg.GdnConfig(2, 32, 16, 128, 128, 64, 4))
    for L in (48, 64):
        with pytest.raises(rb.ReplaySSMError) as e:
            bg.gdn_sizes(bg.GdnConfig(2, 32, 16, 128, 128, L, 8))
        assert e.value.code == -2 and "LDS" in str(e.value)


def test_gdn_null_pointers_rejected_before_launch(rb):
    from mamba_state_replay_amd import binding_gdn as bg
    L = bg.lib()
    c = bg.GdnConfig(4, 32, 16, 128, 128, window=16, max_drafts=2).c()
    s = bg.gdn_state()
    t = bg.gdn_tokens(None, None, None, None, None, 1)
    assert L.gdn_decode_step(ctypes.byref(c), ctypes.byref(s), ctypes.byref(t), None, None) == -1
    assert L.gdn_verify_drafts(ctypes.byref(c), ctypes.byref(s), ctypes.byref(t), None, None) == -1
    assert L.gdn_flush(ctypes.byref(c), ctypes.byref(s), 0, None) == -1
    assert L.gdn_commit(ctypes.byref(c), ctypes.byref(s), None, 3, None) == -4
    assert L.gdn_commit(ctypes.byref(c), ctypes.byref(s), None, 1, None) == -1
    assert L.gdn_conventional_update(ctypes.byref(c), None, 1, None, None, ctypes.byref(t), None, None) == -1
    assert L.gdn_conventional_commit(ctypes.byref(c), None, 1, None, 1, None, None) == -2
    assert L.gdn_conventional_commit(ctypes.byref(c), None, 4, None, 4, None, None) == -4
    assert L.gdn_conventional_commit(ctypes.byref(c), None, 4, None, 3, None, None) == -1
    assert L.gdn_decode_step(None, None, None, None, None) == -1
    assert L.gdn_commit_verify(ctypes.byref(c), ctypes.byref(s), None, 1, ctypes.byref(t), None, None) == -1
    assert L.gdn_commit_verify(ctypes.byref(c), ctypes.byref(s), None, 3, ctypes.byref(t), None, None) == -4
    zero = bg.GdnConfig(0, 32, 16, 128, 128).c()
    assert L.gdn_decode_step(ctypes.byref(zero), None, None, None, None) == 0   # batch 0: nothing to do


def test_missing_library_raises():
    """With no built library every entry point raises at once: there is no
    fallback path (run in a child process so the loaded library of this one
    is left alone)."""
    code = (
        "import pathlib, pytest\n"
        "from mamba_state_replay_amd import binding as rb, binding_gdn as bg\n"
        "rb.LIBRARY = pathlib.Path('/nonexistent/libreplayssm.so')\n"
        "rb._LIB = None\n"
        "bg._LIB = None\n"
        "with pytest.raises(RuntimeError, match='is missing'):\n"
        "    rb.lib()\n"
        "with pytest.raises(RuntimeError, match='is missing'):\n"
        "    bg.gdn_row_blocks(bg.GdnConfig(1, 2, 1, 128, 128, 16, 1, 'bf16'))\n"
        "print('ok')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         cwd=Path(__file__).resolve().parent.parent)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stderr[-1500:]
