"""The bench's command-line contract on the host: more than one GPU is
refused with a message, and with no HIP device it stops at once with a
message (there is no CPU path)."""
import subprocess
import sys
from pathlib import Path

import pytest
import torch

ROOT = Path(__file__).resolve().parent.parent


def _run(*args):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="a HIP device is visible")
def test_no_device_fails_loudly():
    for cfg in ("decode", "gdn"):
        r = _run("--config", cfg)
        assert r.returncode == 1, r.stderr[-500:]
        assert "no CPU path" in r.stderr
        assert r.stdout == ""
