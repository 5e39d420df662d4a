"""Plant plausible mistakes in copies of the oracle source; the pins must catch each.

Each mutant is compiled from a patched copy of oracle/oracle.c into a temporary
directory and exercised in a child process (a mutant may read out of bounds),
so the real oracle is never touched.
"""
import json
import subprocess
import sys
import textwrap
from pathlib import Path

import pytest

from oracle import _build

ROOT = Path(__file__).resolve().parent.parent
SRC = (ROOT / "oracle" / "oracle.c").read_text()

MUTANTS = {
    "decay_sign": ("exp(dtv * A[h])", "exp(-dtv * A[h])"),
    "no_decay": ("decay * Hbh[i * dstate + j] + dtv", "Hbh[i * dstate + j] + dtv"),
    "no_dt_input_scale": ("+ dtv * xt[i] * Bt[j]", "+ xt[i] * Bt[j]"),
    "transposed_outer": ("dtv * xt[i] * Bt[j]", "dtv * xt[j % headdim] * Bt[i % dstate]"),
    "transposed_read": ("acc += Hbh[i * dstate + j] * Ct[j]",
                        "acc += Hbh[(j % headdim) * dstate + (i % dstate)] * Ct[j]"),
    "no_skip": ("yt[i] = acc + D[h] * xt[i];", "yt[i] = acc;"),
    "wrong_skip_head": ("acc + D[h] * xt[i]", "acc + D[0] * xt[i]"),
    "wrong_group": ("return h / (nheads / ngroups);", "return h % ngroups;"),
    "wrong_decay_head": ("exp(dtv * A[h])", "exp(dtv * A[g])"),
    "read_before_update": ("acc += Hbh[i * dstate + j] * Ct[j];",
                           "acc += (Hbh[i * dstate + j] - dtv * xt[i] * Bt[j]) / decay * Ct[j];"),
    "stale_C": ("const double *Ct = C + (tb * ngroups + g) * dstate;",
                "const double *Ct = C + ((t > 0 ? tb - batch : tb) * ngroups + g) * dstate;"),
    "B_from_C": ("const double *Bt = B + (tb * ngroups + g) * dstate;",
                 "const double *Bt = C + (tb * ngroups + g) * dstate;"),
}

RUNNER = textwrap.dedent("""
    import json, sys
    sys.path.insert(0, {root!r})
    from oracle.oracle import Oracle
    from tests import oracle_pins
    o = Oracle({lib!r})
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception:
            failed.append(pin.__name__)
    print(json.dumps(failed))
""")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation anchor for {name} not found in oracle.c"
    src = tmp_path / "oracle_mut.c"
    src.write_text(SRC.replace(old, new, 1))
    lib = _build.build(src, tmp_path / "liboracle_mut.so", werror=False)
    proc = subprocess.run([sys.executable, "-c", RUNNER.format(root=str(ROOT), lib=str(lib))],
                          capture_output=True, text=True, timeout=300)
    if proc.returncode < 0:
        # killed by a signal (an out-of-bounds mutant): detected
        return
    assert proc.returncode == 0, proc.stderr[-2000:]
    failed = json.loads(proc.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"
