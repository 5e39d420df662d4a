"""The algorithmic byte model behind every GB/s and roofline figure
(mamba_state_replay_amd/traffic.py), checked against sums worked out by hand
from the per-call definitions: a non-flush call reads the tile it needs, the
committed records and the token's inputs and writes the output and the new
record; a flushing call reads and writes the FP32 checkpoint once more; the
conventional step reads and writes the whole state (NVIDIA Developer blog
"ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding",
sections "How ReplaySSM represents the state" and "Benefit 1")."""
import numpy as np

from mamba_state_replay_amd import traffic

# the Nemotron-3-style layer of the benchmarks: 128 heads, headdim 64, dstate 128, 8 groups, bf16 inputs
NEMO = (128, 64, 128, 8)


def test_layer_sizes_by_hand():
    sz = traffic.sizes(*NEMO, in_bytes=2)
    assert sz.S == 128 * 64 * 128 * 4 == 4_194_304
    assert sz.S_r == sz.S and sz.S_c == 0
    # x of every head (bf16) + B of every group (bf16) + dt of every head (fp32)
    assert sz.R == 16_384 + 2_048 + 512 == 18_944
    assert sz.TOK == sz.R + 2_048            # the token also brings C of every group
    assert sz.Y == 128 * 64 * 4
    # conventional step per sequence: state read and written, the token's inputs, the output
    assert traffic.conventional_step_bytes(sz, 1) == 8_442_368


def test_read_copy_sizes_by_hand():
    E = 128 * 64 * 128
    assert traffic.sizes(*NEMO, read_copy="bf16").S_r == 2 * E
    assert traffic.sizes(*NEMO, read_copy="e4m3").S_r == E + 128 * 4          # one fp32 scale per head tile
    assert traffic.sizes(*NEMO, read_copy="mxfp4").S_r == E // 2 + E // 32    # 4-bit codes + an E8M0 byte per 32
    assert traffic.sizes(*NEMO, read_copy="mxfp8").S_r == E + E // 32
    sz = traffic.sizes(*NEMO, read_copy="mxfp4", ckpt_bytes=2)
    assert sz.S == 2 * E and sz.S_c == sz.S_r                                  # FP16 checkpoint, copy rewritten


def test_flush_schedule_from_a_full_window():
    """Starting with L committed records, the first call flushes, then every
    L-th: the call that finds n >= L folds first, and each decode call commits
    its token."""
    L = 16
    sched, n_end = traffic.decode_schedule(np.array([L, 3]), L, 40)
    folds0 = [i for i, (_, f) in enumerate(sched) if f[0]]
    assert folds0 == [0, 16, 32]
    assert [int(n[0]) for n, _ in sched[:3]] == [16, 1, 2]
    folds1 = [i for i, (_, f) in enumerate(sched) if f[1]]
    assert folds1 == [13, 29]
    assert n_end.tolist() == [8, 11]


def test_headline_bytes_per_launch_by_hand():
    """Batch 256, L = 16, all sequences in phase: per window one flushing call
    with n = 16 and fifteen non-flush calls with n = 1 .. 15, so per sequence
    and window 16 (S + TOK + R + Y) + S + (16 + 1 + ... + 15) R."""
    sz = traffic.sizes(*NEMO)
    per_window = 16 * (sz.S + sz.TOK + sz.R + sz.Y) + sz.S + (16 + 120) * sz.R
    assert per_window == 75_042_816
    sched, _ = traffic.decode_schedule(np.full(256, 16), 16, 64)
    total = sum(traffic.decode_step_bytes(sz, n, f) for n, f in sched)
    assert total == 4 * 256 * per_window
    assert total // 64 == 1_200_685_056          # the roofline's algorithmic bytes per launch


def test_verify_and_snapshot_bytes_by_hand():
    sz = traffic.sizes(*NEMO)
    T = 3
    n = np.array([5, 16])
    fold = n >= 16
    # non-flush: the tile, 5 records, and per draft its inputs, its record and its output
    nonfold = sz.S + 5 * sz.R + T * (sz.TOK + sz.R + sz.Y)
    # flushing: the checkpoint read and written, 16 records, the drafts
    folded = 2 * sz.S + 16 * sz.R + T * (sz.TOK + sz.R + sz.Y)
    assert traffic.verify_bytes(sz, n, fold, T) == nonfold + folded
    # snapshots: the state read once and one snapshot written per draft
    assert traffic.snapshot_verify_bytes(sz, 2, T) == 2 * (4 * sz.S + T * (sz.TOK + sz.Y))


def test_gdn_sizes_by_hand():
    sz = traffic.gdn_sizes(32, 16, 128, 128)
    assert sz.S == 32 * 128 * 128 * 4 == 2_097_152
    # a record: the key of every key head (bf16), u of every value head (fp32), g (fp32)
    assert sz.R == 4_096 + 16_384 + 128
    # a token: q and k of every key head (bf16), v of every value head (bf16), g and beta (fp32)
    assert sz.TOK == 8_192 + 8_192 + 256
    assert sz.Y == 32 * 128 * 4
    assert traffic.gdn_sizes(32, 16, 128, 128, ckpt_bytes=2).S == sz.S // 2
