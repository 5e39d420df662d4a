"""The oracle's scenario functions against brute force and the replay model,
and planted mistakes in copies of oracle/oracle.py that those pins must catch.

A mutant is the oracle module's source with one plausible slip patched in,
loaded as a separate module under another name (the real module is never
touched); its functions still step the real fp64 library.
"""
import importlib.util
import sys
from pathlib import Path

import pytest

from tests import scenario_pins

ROOT = Path(__file__).resolve().parent.parent
SRC = (ROOT / "oracle" / "oracle.py").read_text()

MUTANTS = {
    # the commit of round r takes the next round's accepted counts
    "commit_next_round": ("nsteps=acc[r][sl]", "nsteps=acc[min(r + 1, len(acc) - 1)][sl]"),
    # every draft committed, whatever was accepted
    "commit_all_drafts": ("nsteps=acc[r][sl]", "nsteps=None"),
    # round r's drafts read one token late
    "draft_slice_off_by_one": ("_tok(work.steps, r * T, r * T + T, seqs)",
                               "_tok(work.steps, r * T + 1, r * T + T + 1, seqs)"),
    # the committed record counts of another sequence
    "other_sequence_n0": ("n0 = work.n0[sl]", "n0 = np.roll(work.n0, 1)[sl]"),
    # every pre-filled record counted as committed
    "all_records_committed": ("nsteps=n0,", "nsteps=None,"),
    # the committed state built from zero instead of the checkpoint
    "zero_checkpoint": ("h0 = work.h0[sl]", "h0 = 0 * work.h0[sl]"),
    # decode tokens read from the second one on
    "decode_skips_token": ("H = committed_state(work, seqs, orc, threads)\n    x, B, C, dt = _tok(work.steps, 0, nsteps, seqs)",
                           "H = committed_state(work, seqs, orc, threads)\n    x, B, C, dt = _tok(work.steps, 1, nsteps + 1, seqs)"),
    # decode starts from the checkpoint, ignoring the committed records
    "decode_ignores_records": ("H = committed_state(work, seqs, orc, threads)\n    x, B, C, dt = _tok(work.steps, 0, nsteps, seqs)",
                               "H = work.h0[slice(None) if seqs is None else seqs]\n    x, B, C, dt = _tok(work.steps, 0, nsteps, seqs)"),
    # the drafts' outputs read from the state after the commit of the same round
    "verify_outputs_after_commit": (
        "_, y = orc.conventional(H, x, B, C, dt, work.A, work.D, threads=threads)\n        ys.append(y)\n        H, _ = orc.conventional(H, x, B, C, dt, work.A, work.D,\n                                nsteps=acc[r][sl], outputs=False, threads=threads)",
        "H, _ = orc.conventional(H, x, B, C, dt, work.A, work.D,\n                                nsteps=acc[r][sl], outputs=False, threads=threads)\n        _, y = orc.conventional(H, x, B, C, dt, work.A, work.D, threads=threads)\n        ys.append(y)"),
    # the selected sequences' tokens not selected
    "tokens_ignore_selection": ("sl = slice(None) if seqs is None else seqs\n    return (tokens",
                                "sl = slice(None)\n    return (tokens"),
}


def _load(name, src, tmp_path):
    path = tmp_path / f"{name}.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    try:
        spec.loader.exec_module(mod)
    finally:
        sys.modules.pop(spec.name, None)
    return mod


@pytest.mark.parametrize("pin", scenario_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_scenario_pin(orc, pin):
    from oracle import oracle as om
    pin(om, orc)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_scenario_mutant_is_caught(orc, tmp_path, name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not found once in oracle.py"
    mod = _load(name, SRC.replace(old, new), tmp_path)
    failed = []
    for pin in scenario_pins.ALL_PINS:
        try:
            pin(mod, orc)
        except Exception:            # a wrong value, a wrong shape or a crash all count
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every scenario pin"
