"""Build libreplayssm.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m mamba_state_replay_amd._build
Always recompiles.  Objects go to mamba_state_replay_amd/_build/ (ignored).
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
ROOT = PKG.parent
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libreplayssm.so"
OBJDIR = PKG / "_build"

ARCH = "gfx950"
SOURCES = ["replay.hip", "replay_f16.hip", "conventional.hip", "gdn.hip", "probe.hip", "api.cpp"]

# Packed fp32 instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise FileNotFoundError("hipcc not found (set HIPCC)")


def _compile(src: Path, obj: Path, extra: list[str]) -> None:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
           f"-I{INCLUDE}", "-c", str(src), "-o", str(obj)] + DEVICE_FLAGS + extra
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{proc.stderr}")


def build(extra: list[str] | None = None, jobs: int = 5) -> Path:
    """Compile every source and link libreplayssm.so; returns its path."""
    extra = list(extra or [])
    OBJDIR.mkdir(exist_ok=True)
    srcs = [CSRC / s for s in SOURCES]
    objs = [OBJDIR / (s.name + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(srcs, objs)))
    tmp = LIBRARY.with_name(LIBRARY.name + f".tmp{os.getpid()}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp)] + [str(o) for o in objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
