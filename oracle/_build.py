"""Compile the C oracle into oracle/liboracle.so with the host C compiler.

Test infrastructure: the HIP library never links or loads the result.
"""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "oracle.c"
LIBRARY = HERE / "liboracle.so"


def build(src: Path | str = SOURCE, out: Path | str = LIBRARY, cc: str | None = None,
          werror: bool = True) -> Path:
    """Build `src` into the shared library `out` (always recompiles)."""
    cc = cc or os.environ.get("CC", "gcc")
    out = Path(out)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = [cc, "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall"] + (["-Werror"] if werror else []) + [
           str(src), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
