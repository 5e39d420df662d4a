#!/usr/bin/env python3
"""Benchmark of the ReplaySSM decode hot path on one MI355X.

Workload: the Nemotron-3-style Mamba-2 layer (batch 256, nheads 128, headdim
64, dstate 128, ngroups 8; FP32 state 4 MiB per sequence), window L = 16, bf16
x/B/C and fp32 dt, seeded synthetic inputs, steady state (every sequence starts
with L committed records, so one call in 16 flushes).  One step = one
replayssm_decode_step call over the whole batch, flush included when due.

Prints one JSON line: value = achieved algorithmic HBM GB/s of the decode step
(ms_per_step carries the time), the roofline of the replay kernel, the
in-library conventional kernel on the same inputs, the streaming-probe ceiling
and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "Mamba-2 layer decode-step µs + achieved HBM GB/s at batch 256, L=16"
PEAK_GBS = 8000.0
COUNTERS = ROOT / "profiles" / "replay_decode_batch256_L16_counters.json"
KERNEL_SOURCES = ["mamba_state_replay_amd/csrc/replay.hip", "mamba_state_replay_amd/csrc/replay_impl.h",
                  "mamba_state_replay_amd/csrc/common.h"]


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update((ROOT / p).read_bytes())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--window", type=int, default=16)
    ap.add_argument("--read-copy", choices=["none", "bf16", "e4m3", "mxfp4", "mxfp8"], default="none")
    ap.add_argument("--stagger", action="store_true",
                    help="staggered phases: sequence b starts with 1 + (b mod L) committed records, so about "
                         "1/L of the sequences flush in every step (default: all start with L and flush together)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-conventional", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="decode: skip the other workloads measured after the headline (verification at "
                         "batch 512 with T = 3 and 8, the read copies and FP16 checkpoint, the GDN layer)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the CPU sample")
    ap.add_argument("--config", choices=["decode", "verify", "verify_sweep", "sweep", "dual", "gdn",
                                         "gdn_verify_sweep", "gdn_sweep"], default="decode",
                    help="decode: the headline line (default); verify: speculative rounds at batch 512, "
                         "T=3; verify_sweep: the same for T in 1, 2, 3, 4, 8; sweep: batch x window grid; "
                         "dual: FP32 / bf16 / e4m3 read copies over 4096 steps; gdn: Gated DeltaNet layer "
                         "decode and verify (batch --gdn-batch)")
    ap.add_argument("--gdn-batch", type=int, default=512)
    ap.add_argument("--gdn-ckpt", choices=["f32", "f16"], default="f32",
                    help="GDN checkpoint: FP32, or FP16 written with stochastic rounding")
    ap.add_argument("--summarize-configs", nargs="+", metavar="LOG",
                    help="write the tables of bench logs of the non-default configs into profiles/ and exit")
    ap.add_argument("--ingest-gdn-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="summarise rocprofv3 output of the GDN runs into profiles/ and exit")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="summarise rocprofv3 output of the counter runs into profiles/ and exit")
    ap.add_argument("--ingest-sq-counters", action="store_true",
                    help="summarise the rocprofv3 runs of SQ_PROFILE_CMDS (MXFP4 copy HBM and SQ counters, "
                         "FP32 SQ counters) into profiles/ and exit")
    return ap.parse_args()


def timed_launches(fn, steps, torch):
    """Run fn(i) for i < steps with an event pair around each launch.

    Returns (total ms of the region, list of per-launch ms)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    region0.record()
    for i in range(steps):
        starts[i].record()
        fn(i)
        ends[i].record()
    region1.record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return region0.elapsed_time(region1), per


def graph_time(fn, steps, torch):
    """Capture fn(0) .. fn(steps-1) in one HIP graph (torch.cuda.graph) and time
    one replay after a warm one: GPU time of the launches without the host's
    per-launch cost.  Returns ms for all steps."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_sq_counters:
        ingest_sq_counters()
        return
    if args.ingest_gdn_counters:
        ingest_gdn_counters(*args.ingest_gdn_counters)
        return
    if args.summarize_configs:
        summarize_configs(args.summarize_configs)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path shards by sequence or head group with no "
              "exchange, so only --gpus 1 is run here.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py times the HIP kernels on an MI355X and has no CPU path: no HIP device is "
              "visible.", file=sys.stderr)
        sys.exit(1)
    if args.config != "decode":
        {"verify": bench_verify, "verify_sweep": bench_verify_sweep, "sweep": bench_sweep,
         "dual": bench_dual, "gdn": bench_gdn, "gdn_verify_sweep": bench_gdn_verify_sweep,
         "gdn_sweep": bench_gdn_sweep}[args.config](args)
        return

    from mamba_state_replay_amd import binding as rb
    from mamba_state_replay_amd import staging, synth, traffic

    dev = torch.device("cuda", 0)
    L = args.window
    read_copy = None if args.read_copy == "none" else args.read_copy
    shape = synth.LayerShape(batch=args.batch, nheads=128, headdim=64, dstate=128, ngroups=8, window=L)
    ntok = 64
    work = synth.decode_workload(shape, ntok, seed=1001,
                                 n0=synth.staggered_fill(shape.batch, L) if args.stagger else L)
    cfg = staging.config(shape, read_copy=read_copy)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    toks = staging.TokenStream(work.steps, dev)
    y = torch.empty((shape.batch, 1, shape.nheads, shape.headdim), device=dev)
    if read_copy:
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)

    W, K = args.warmup, args.steps
    for i in range(W):
        rb.replayssm_decode_step(cfg, st, p, toks.call(i % ntok), y)
    torch.cuda.synchronize()

    # Three passes of K steps after the warm-up: eager launches with an event
    # pair around each (the kernel's own duration), then the same K launches
    # captured in one HIP graph, replayed once to warm up and once timed (the
    # step time without the host's per-launch cost, as a decode loop runs them).
    sched, n_end = traffic.decode_schedule(work.n0, L, W + 3 * K)
    sz = traffic.sizes(128, 64, 128, 8, 2, read_copy)
    eager_sched = sched[W:W + K]
    graph_sched = sched[W + 2 * K:W + 3 * K]
    bytes_per_launch = [traffic.decode_step_bytes(sz, n, f) for n, f in eager_sched]
    folds = sum(int(f.any()) for _, f in graph_sched)

    step = lambda i: rb.replayssm_decode_step(cfg, st, p, toks.call((W + i) % ntok), y)
    eager_ms, per_ms = timed_launches(step, K, torch)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            rb.replayssm_decode_step(cfg, st, p, toks.call((W + K + i) % ntok), y)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    del g
    # Steady state beside the K-step figure: a whole number of windows (one
    # flush per L calls exactly), captured and timed the same way, so the
    # µs/step does not depend on how K lines up with L.
    ss_steps = L * max(1, -(-64 // L))
    ss_first = W + 3 * K
    ss_ms = graph_time(lambda i: rb.replayssm_decode_step(cfg, st, p, toks.call((ss_first + i) % ntok), y),
                       ss_steps, torch)
    # graph_time replays the capture twice (a warm replay, then the timed one)
    ss_sched, n_end = traffic.decode_schedule(work.n0, L, ss_first + 2 * ss_steps)
    ss_sched = ss_sched[ss_first + ss_steps:]
    ss_bytes = sum(traffic.decode_step_bytes(sz, n, f) for n, f in ss_sched)
    ss_folds = sum(int(f.any()) for _, f in ss_sched)
    meta = st.meta.cpu().numpy()
    assert np.all(meta[:, :, 1] == n_end[:, None]), "ring pointers disagree with the flush schedule"
    assert int(st.status.cpu()[0]) == 0 and bool(torch.isfinite(y).all())

    total_bytes = sum(traffic.decode_step_bytes(sz, n, f) for n, f in graph_sched)
    us_step = total_ms * 1e3 / K
    gbs = total_bytes / (total_ms * 1e-3) / 1e9
    kernel_ms = float(np.mean(per_ms))
    achieved = (sum(bytes_per_launch) / K) / (kernel_ms * 1e-3) / 1e9
    fold_ms = [t for t, (_, f) in zip(per_ms, eager_sched) if f.any()]
    nonfold_ms = [t for t, (_, f) in zip(per_ms, eager_sched) if not f.any()]

    traffic_bytes = None
    if COUNTERS.exists():
        c = json.loads(COUNTERS.read_text())
        if (c.get("source_hash") == source_hash(KERNEL_SOURCES) and c.get("batch") == shape.batch
                and c.get("window") == L and read_copy is None and not args.stagger):
            traffic_bytes = c.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(total_ms / K, 6),
        "us_per_step": round(us_step, 2),
        "timing": "K steps captured in one HIP graph, one replay timed with HIP events after a warm replay",
        "eager_us_per_step": round(eager_ms * 1e3 / K, 2),
        "steady_state": {"us_per_step": round(ss_ms * 1e3 / ss_steps, 2),
                         "gbs": round(ss_bytes / (ss_ms * 1e-3) / 1e9, 1),
                         "steps": ss_steps, "flush_calls": ss_folds,
                         "note": "a whole number of windows, one flushing call per L (graph-timed)"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"Nemotron-3-style Mamba-2 layer decode (ReplaySSM), batch {shape.batch}, "
                        f"nheads 128, headdim 64, dstate 128, ngroups 8, L={L}, bf16 x/B/C, fp32 dt, "
                        f"FP32 checkpoint" + (f" + {read_copy} read copy" if read_copy else "") +
                        (", staggered phases (1 + b mod L committed records at start)" if args.stagger else
                         ", steady state (L committed records at start)"),
            "batch": shape.batch, "window": L, "read_copy": read_copy or "none",
            "phases": "staggered" if args.stagger else "aligned",
            "flush_launches_timed": folds,
        },
        "kernel_source_hash": source_hash(KERNEL_SOURCES),
        "roofline": {
            "bound": "hbm",
            "kernel": "replay_kernel",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic_bytes,
            "algorithmic_bytes_per_launch": int(sum(bytes_per_launch) / K),
            "avg_launch_us": round(kernel_ms * 1e3, 2),
            "nonflush_launch_us": round(float(np.mean(nonfold_ms)) * 1e3, 2) if nonfold_ms else None,
            "flush_launch_us": round(float(np.mean(fold_ms)) * 1e3, 2) if fold_ms else None,
        },
    }

    if not args.no_conventional:
        states = staging.conventional_states(cfg, work.h0, 1, dev)
        for i in range(W):
            rb.conventional_state_update(cfg, states, p, toks.call(i % ntok), y)
        cstep = lambda i: rb.conventional_state_update(cfg, states, p, toks.call((W + i) % ntok), y)
        ceager, cper = timed_launches(cstep, K, torch)
        ctot = graph_time(cstep, K, torch)
        cbytes = traffic.conventional_step_bytes(sz, shape.batch)
        c_us = ctot * 1e3 / K
        result["conventional"] = {
            "us_per_step": round(c_us, 2),
            "eager_us_per_step": round(ceager * 1e3 / K, 2),
            "gbs": round(cbytes / (c_us * 1e-6) / 1e9, 1),
            "avg_launch_us": round(float(np.mean(cper)) * 1e3, 2),
            "frac": round(cbytes / (float(np.mean(cper)) * 1e-3) / 1e9 / PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": cbytes,
        }
        result["speedup_vs_conventional"] = round(c_us / us_step, 3)
        del states

    if not args.no_probe:
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
        dst = torch.empty_like(src)
        sink = torch.zeros(rb.probe_sink_elems(nbytes), dtype=torch.float32, device=dev)
        for _ in range(3):
            rb.rssm_probe_read(src, sink)
            rb.rssm_probe_copy(dst, src)
        rt, rper = timed_launches(lambda i: rb.rssm_probe_read(src, sink), 10, torch)
        ct, cper = timed_launches(lambda i: rb.rssm_probe_copy(dst, src), 10, torch)
        read_gbs = nbytes / (float(np.median(rper)) * 1e-3) / 1e9
        copy_gbs = 2 * nbytes / (float(np.median(cper)) * 1e-3) / 1e9
        result["probe"] = {"read_gbs": round(read_gbs, 1), "copy_gbs": round(copy_gbs, 1),
                           "bytes": nbytes}
        result["roofline"]["frac_of_probe_read"] = round(achieved / read_gbs, 4)
        del src, dst, sink

    if not args.no_extras:
        result["also"] = extras(args)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(work, total_bytes / K, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def extras(args):
    """The other workloads, measured after the headline in the same run, each
    in compact form (the --config runs give the full records): speculative
    verification at batch 512 (T = 3 and 8, replay against FP32 snapshots),
    decode with each read copy and with the FP16 checkpoint (batch 256,
    L = 16, 256 steps = 16 whole windows), and the GDN layer (batch 512,
    decode and T = 3 verification).  Times are graph-timed as in the --config
    runs; launch times are HIP event pairs around eager launches."""
    import torch
    import traceback

    def verify(T):
        pt = _verify_point(T, rounds=32)
        return {"replay_us_per_round": pt["replay"]["us_per_round"], "replay_gbs": pt["replay"]["gbs"],
                "fused_commit_us_per_round": pt["replay_fused_commit"]["us_per_round"],
                "snapshot_us_per_round": pt["snapshot_baseline"]["us_per_round"],
                "speedup_vs_snapshot": pt["speedup"], "rounds": 32}

    def gdn():
        g = gdn_measure(argparse.Namespace(window=16, gdn_batch=512, gdn_ckpt="f32", steps=64, warmup=16,
                                           no_probe=True, no_cpu=True))
        return {"us_per_step": g["us_per_step"], "gbs": g["value"],
                "nonflush_launch_us": g["roofline"]["nonflush_launch_us"],
                "flush_launch_us": g["roofline"]["flush_launch_us"],
                "conventional_us_per_step": g["conventional"]["us_per_step"],
                "speedup_vs_conventional": g["speedup_vs_conventional"],
                "verify_T3_us_per_round": g["verify_T3"]["us_per_round"],
                "snapshot_T3_us_per_round": g["verify_T3"]["snapshot_baseline_us_per_round"],
                "speedup_vs_snapshot": g["verify_T3"]["speedup_vs_snapshot"]}

    out = {}
    jobs = [("verify_batch512_T3", lambda: verify(3)), ("verify_batch512_T8", lambda: verify(8)),
            ("read_copies_batch256_L16", lambda: {"steps": 256, "modes": dual_measure(256)}),
            ("gdn_batch512_L16", gdn)]
    for key, fn in jobs:
        torch.cuda.empty_cache()
        try:
            out[key] = fn()
        except Exception as e:          # a failed extra is reported in its place; the headline stands
            traceback.print_exc()
            out[key] = {"error": f"{type(e).__name__}: {e}"}
    torch.cuda.empty_cache()
    return out


GDN_LAYER = dict(nv=32, nk=16, dk=128, dv=128)


def bench_gdn(args):
    """Gated DeltaNet layer (32 value heads over 16 key heads, dk = dv = 128,
    FP32 state 2 MiB per sequence), batch --gdn-batch, L = --window: replay
    decode steps (steady state reached from an empty buffer during the
    warm-up) against the in-library conventional GDN step, then speculative
    rounds of T = 3 drafts with U{0..3} acceptance; one JSON line."""
    print(json.dumps(gdn_measure(args)), flush=True)


def gdn_measure(args):
    """The measurements of bench_gdn, returned as its record."""
    torch, dev = _device()
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd import staging, synth_gdn, traffic

    L, batch = args.window, args.gdn_batch
    shape = synth_gdn.GdnShape(batch=batch, window=L, **GDN_LAYER)
    ntok = 32
    w = synth_gdn.gdn_workload(shape, ntok, seed=2001)
    ck = args.gdn_ckpt
    cfg = bg.GdnConfig(batch, shape.nv, shape.nk, shape.dk, shape.dv, L, 1, "bf16", ck)
    st = bg.GdnState.allocate(cfg, dev)
    st.ckpt.copy_(torch.from_numpy(w.S0).to(dev).to(cfg.ckpt_torch))
    toks = staging.GdnTokenStream(w.steps, dev)
    o = torch.empty((batch, 1, shape.nv, shape.dv), device=dev)
    sz = traffic.gdn_sizes(shape.nv, shape.nk, shape.dk, shape.dv, ckpt_bytes=2 if ck == "f16" else 4)
    csz = traffic.gdn_sizes(shape.nv, shape.nk, shape.dk, shape.dv)
    W, K = max(args.warmup, L + 1), args.steps
    for i in range(W):
        bg.gdn_decode_step(cfg, st, toks.call(i % ntok), o)
    sched, n_end = traffic.decode_schedule(np.zeros(batch, np.int64), L, W + 3 * K)
    eager_sched, graph_sched = sched[W:W + K], sched[W + 2 * K:W + 3 * K]
    step = lambda i: bg.gdn_decode_step(cfg, st, toks.call((W + i) % ntok), o)
    eager_ms, per_ms = timed_launches(step, K, torch)
    total_ms = graph_time(lambda i: bg.gdn_decode_step(cfg, st, toks.call((W + K + i) % ntok), o), K, torch)
    meta = st.meta.cpu().numpy()
    assert np.all(meta[..., 1] == n_end[:, None, None]), "ring pointers disagree with the flush schedule"
    assert int(st.status.cpu()[0]) == 0 and bool(torch.isfinite(o).all())
    launch_bytes = [traffic.decode_step_bytes(sz, n, f) for n, f in eager_sched]
    step_bytes = sum(traffic.decode_step_bytes(sz, n, f) for n, f in graph_sched) / K
    kernel_ms = float(np.mean(per_ms))
    achieved = float(np.mean(launch_bytes)) / (kernel_ms * 1e-3) / 1e9
    fold_ms = [t for t, (_, f) in zip(per_ms, eager_sched) if f.any()]
    nonfold_ms = [t for t, (_, f) in zip(per_ms, eager_sched) if not f.any()]
    us_step = total_ms * 1e3 / K
    gdn_hash = source_hash(["mamba_state_replay_amd/csrc/gdn.hip", "mamba_state_replay_amd/csrc/common.h"])
    gdn_counters = ROOT / "profiles" / "gdn_decode_batch512_L16_counters.json"
    traffic_bytes = None
    if gdn_counters.exists():
        c = json.loads(gdn_counters.read_text())
        if c.get("source_hash") == gdn_hash and c.get("batch") == batch and c.get("window") == L and ck == "f32":
            traffic_bytes = c.get("bytes_per_launch")

    S = torch.from_numpy(w.S0).to(dev)
    ccfg = bg.GdnConfig(batch, shape.nv, shape.nk, shape.dk, shape.dv, L, 1, "bf16")   # FP32 state
    cstep = lambda i: bg.gdn_conventional_update(ccfg, S, toks.call(i % ntok), o)  # nslots 1: in place
    for i in range(4):
        cstep(i)
    ceager, cper = timed_launches(cstep, K, torch)
    ctot = graph_time(cstep, K, torch)
    cbytes = traffic.conventional_step_bytes(csz, batch)
    c_us = ctot * 1e3 / K
    del S

    # snapshot verification baseline: T = 3 drafts, one FP32 state snapshot per draft
    T = 3
    snap = torch.empty((batch, T + 1, shape.nv, shape.dv, shape.dk), device=dev)
    snap[:, 0] = torch.from_numpy(w.S0).to(dev)
    slot = torch.zeros(batch, dtype=torch.int32, device=dev)
    # speculative rounds: T = 3 drafts, U{0..3} accepted, verify + commit
    rounds = 32
    vw = synth_gdn.gdn_workload(shape, rounds, seed=2003, T=T, ckpt_std=0.0)
    vcfg = bg.GdnConfig(batch, shape.nv, shape.nk, shape.dk, shape.dv, L, T, "bf16", ck)
    scfg = bg.GdnConfig(batch, shape.nv, shape.nk, shape.dk, shape.dv, L, T, "bf16")
    del st, toks
    vst = bg.GdnState.allocate(vcfg, dev)
    vst.ckpt.copy_(torch.from_numpy(w.S0).to(dev).to(vcfg.ckpt_torch))
    vtoks = staging.GdnTokenStream(vw.steps, dev, T)
    acc = torch.from_numpy(vw.extra["accepted"]).to(dev)
    vo = torch.empty((batch, T, shape.nv, shape.dv), device=dev)
    vround = lambda r: (bg.gdn_verify_drafts(vcfg, vst, vtoks.call(r % rounds), vo),
                        bg.gdn_commit(vcfg, vst, acc[r % rounds], T))
    for r in range(8):
        vround(r)
    v_ms = graph_time(lambda r: vround(8 + r), rounds, torch)
    assert int(vst.status.cpu()[0]) == 0 and bool(torch.isfinite(vo).all())
    # the commit of round r - 1 fused into the verification of round r: one launch per round,
    # after a verification of round 39 that nothing has committed yet (every round above ended
    # with its commit)
    fround = lambda r: bg.gdn_commit_verify(vcfg, vst, acc[(r - 1) % rounds], T, vtoks.call(r % rounds), vo)
    bg.gdn_verify_drafts(vcfg, vst, vtoks.call(39 % rounds), vo)
    for r in range(4):
        fround(40 + r)
    f_ms = graph_time(lambda r: fround(44 + r), rounds, torch)
    assert int(vst.status.cpu()[0]) == 0 and bool(torch.isfinite(vo).all())
    sround = lambda r: (bg.gdn_conventional_update(scfg, snap, vtoks.call(r % rounds), vo, nslots=T + 1, slot=slot),
                        bg.gdn_conventional_commit(scfg, slot, T + 1, acc[r % rounds], T))
    for r in range(4):
        sround(r)
    s_ms = graph_time(lambda r: sround(4 + r), rounds, torch)
    assert bool(torch.isfinite(vo).all())
    del snap

    result = {
        "metric": "GDN layer decode-step us + achieved HBM GB/s",
        "value": round(step_bytes / (us_step * 1e-6) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(total_ms / K, 6),
        "us_per_step": round(us_step, 2),
        "timing": "K steps captured in one HIP graph, one replay timed with HIP events after a warm replay",
        "eager_us_per_step": round(eager_ms * 1e3 / K, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"Gated DeltaNet layer decode (ReplaySSM), batch {batch}, 32 value heads over 16 "
                               f"key heads, dk = dv = 128, L={L}, bf16 q/k/v, fp32 g/beta, " +
                               ("FP32 checkpoint (2 MiB per sequence)" if ck == "f32" else
                                "FP16 checkpoint with stochastic rounding (1 MiB per sequence)") + ", steady state",
                   "batch": batch, "window": L, "ckpt": ck, "flush_launches_timed": len(fold_ms)},
        "kernel_source_hash": gdn_hash,
        "roofline": {"bound": "hbm", "kernel": "gdn_replay_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic_bytes, "algorithmic_bytes_per_launch": int(np.mean(launch_bytes)),
                     "avg_launch_us": round(kernel_ms * 1e3, 2),
                     "nonflush_launch_us": round(float(np.mean(nonfold_ms)) * 1e3, 2) if nonfold_ms else None,
                     "flush_launch_us": round(float(np.mean(fold_ms)) * 1e3, 2) if fold_ms else None},
        "conventional": {"us_per_step": round(c_us, 2), "eager_us_per_step": round(ceager * 1e3 / K, 2),
                         "gbs": round(cbytes / (c_us * 1e-6) / 1e9, 1),
                         "avg_launch_us": round(float(np.mean(cper)) * 1e3, 2),
                         "frac": round(cbytes / (float(np.mean(cper)) * 1e-3) / 1e9 / PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": cbytes},
        "speedup_vs_conventional": round(c_us / us_step, 3),
        "verify_T3": {"us_per_round": round(v_ms * 1e3 / rounds, 2), "rounds": rounds,
                      "fused_commit_us_per_round": round(f_ms * 1e3 / rounds, 2),
                      "snapshot_baseline_us_per_round": round(s_ms * 1e3 / rounds, 2),
                      "snapshot_baseline_state": "FP32",
                      "speedup_vs_snapshot": round(s_ms / v_ms, 3),
                      "algorithmic_bytes_snapshot_per_round": traffic.snapshot_verify_bytes(csz, batch, T),
                      "note": "verify + commit per round vs the conventional kernel writing one FP32 snapshot "
                              "per draft + slot commit, both graph-timed"},
    }
    if not args.no_probe:
        from mamba_state_replay_amd import binding as rb
        vst = vtoks = None
        torch.cuda.empty_cache()
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            rb.rssm_probe_copy(dst, src)
        _, cper = timed_launches(lambda i: rb.rssm_probe_copy(dst, src), 10, torch)
        copy_gbs = 2 * nbytes / (float(np.median(cper)) * 1e-3) / 1e9
        result["probe"] = {"copy_gbs": round(copy_gbs, 1), "bytes": nbytes}
        del src, dst
    if not args.no_cpu:
        result["cpu_baseline"] = gdn_cpu_baseline(w, step_bytes, args.cpu_seconds)
    del vst, vtoks
    torch.cuda.empty_cache()
    return result


def bench_gdn_verify_sweep(args):
    """GDN speculative rounds at batch --gdn-batch, L = 16, for T = 1, 2, 3, 4, 8:
    replay verify + commit against the conventional GDN kernel writing one FP32
    snapshot per draft + slot commit (both graph-timed, 8 rounds of seeded
    drafts with U{0..T} acceptance cycled); one JSON line with the table."""
    torch, dev = _device()
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd import staging, synth_gdn, traffic

    batch, L = args.gdn_batch, args.window
    rows = []
    for T in (1, 2, 3, 4, 8):
        shape = synth_gdn.GdnShape(batch=batch, window=L, max_drafts=T, **GDN_LAYER)
        R = 8
        w = synth_gdn.gdn_workload(shape, R, seed=2100 + T, T=T)
        cfg = bg.GdnConfig(batch, shape.nv, shape.nk, shape.dk, shape.dv, L, T, "bf16")
        st = bg.GdnState.allocate(cfg, dev)
        st.ckpt.copy_(torch.from_numpy(w.S0).to(dev))
        toks = staging.GdnTokenStream(w.steps, dev, T)
        acc = torch.from_numpy(w.extra["accepted"]).to(dev)
        o = torch.empty((batch, T, shape.nv, shape.dv), device=dev)
        rnd = lambda r: (bg.gdn_verify_drafts(cfg, st, toks.call(r % R), o), bg.gdn_commit(cfg, st, acc[r % R], T))
        for r in range(2 * R):
            rnd(r)
        K = 32
        rep_ms = graph_time(lambda r: rnd(r), K, torch)
        assert int(st.status.cpu()[0]) == 0 and bool(torch.isfinite(o).all())
        del st
        snap = torch.empty((batch, T + 1, shape.nv, shape.dv, shape.dk), device=dev)
        snap[:, 0] = torch.from_numpy(w.S0).to(dev)
        slot = torch.zeros(batch, dtype=torch.int32, device=dev)
        srnd = lambda r: (bg.gdn_conventional_update(cfg, snap, toks.call(r % R), o, nslots=T + 1, slot=slot),
                          bg.gdn_conventional_commit(cfg, slot, T + 1, acc[r % R], T))
        for r in range(4):
            srnd(r)
        snap_ms = graph_time(lambda r: srnd(r), K, torch)
        sz = traffic.gdn_sizes(shape.nv, shape.nk, shape.dk, shape.dv)
        del snap, toks
        rows.append({"T": T, "replay_us_per_round": round(rep_ms * 1e3 / K, 2),
                     "snapshot_us_per_round": round(snap_ms * 1e3 / K, 2),
                     "speedup": round(snap_ms / rep_ms, 3),
                     "snapshot_algorithmic_gb_per_round": round(traffic.snapshot_verify_bytes(sz, batch, T) / 1e9, 3)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"config": "gdn_verify_sweep", "batch": batch, "window": L,
                      "workload": "Gated DeltaNet layer, 32 value heads over 16 key heads, dk = dv = 128, bf16 "
                                  "inputs, FP32 checkpoint; U{0..T} acceptance",
                      "timing": "32 rounds captured in one HIP graph, one replay timed after a warm replay",
                      "rows": rows}), flush=True)


def bench_gdn_sweep(args):
    """GDN decode at batch 16, 64, 256 and 512 (L = --window): replay decode
    steps against the conventional GDN step, both graph-timed.  Below about
    1 GiB of state, R replicas of the layer's state are rotated (call i uses
    replica i mod R) so that the steps stream from HBM rather than the 256 MB
    Infinity Cache; each replica runs 16 steps after a 17-step warm-up (one
    flush each).  One JSON line with the table."""
    torch, dev = _device()
    from mamba_state_replay_amd import binding_gdn as bg
    from mamba_state_replay_amd import staging, synth_gdn, traffic

    L = args.window
    rows = []
    for batch in (16, 64, 256, 512):
        shape = synth_gdn.GdnShape(batch=batch, window=L, **GDN_LAYER)
        state_bytes = batch * shape.nv * shape.dv * shape.dk * 4
        R = max(1, -(-(1 << 30) // state_bytes))
        w = synth_gdn.gdn_workload(shape, 32, seed=2200 + batch)
        cfg = bg.GdnConfig(batch, shape.nv, shape.nk, shape.dk, shape.dv, L, 1, "bf16")
        toks = staging.GdnTokenStream(w.steps, dev)
        S0 = torch.from_numpy(w.S0).to(dev)
        sts = []
        for _ in range(R):
            st = bg.GdnState.allocate(cfg, dev)
            st.ckpt.copy_(S0)
            sts.append(st)
        o = torch.empty((batch, 1, shape.nv, shape.dv), device=dev)
        step = lambda i: bg.gdn_decode_step(cfg, sts[i % R], toks.call((i // R) % 32), o)
        W = 17 * R
        for i in range(W):
            step(i)
        K = 16 * R
        rep_ms = graph_time(lambda i: step(W + i), K, torch)
        assert all(int(st.status.cpu()[0]) == 0 for st in sts)
        del sts
        convs = [S0.clone() for _ in range(R)]
        cstep = lambda i: bg.gdn_conventional_update(cfg, convs[i % R], toks.call((i // R) % 32), o)
        for i in range(R):
            cstep(i)
        conv_ms = graph_time(cstep, K, torch)
        del convs, toks, S0
        sz = traffic.gdn_sizes(shape.nv, shape.nk, shape.dk, shape.dv)
        sched, _ = traffic.decode_schedule(np.zeros(batch, np.int64), L, 17 + 16)
        alg = sum(traffic.decode_step_bytes(sz, n, f) for n, f in sched[17:]) / 16
        r_us, c_us = rep_ms * 1e3 / K, conv_ms * 1e3 / K
        rows.append({"batch": batch, "replicas": R, "replay_us_per_step": round(r_us, 2),
                     "conventional_us_per_step": round(c_us, 2), "speedup": round(c_us / r_us, 3),
                     "replay_gbs": round(alg / (r_us * 1e-6) / 1e9, 1),
                     "conventional_gbs": round(traffic.conventional_step_bytes(sz, batch) / (c_us * 1e-6) / 1e9, 1)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"config": "gdn_sweep", "window": L,
                      "workload": "Gated DeltaNet layer, 32 value heads over 16 key heads, dk = dv = 128, bf16 "
                                  "inputs, FP32 checkpoint, steady state from an empty buffer",
                      "timing": "16 steps per replica captured in one HIP graph, one replay timed after a warm one",
                      "rows": rows}), flush=True)


def gdn_cpu_baseline(w, gpu_bytes_per_step, target_s):
    """The fp64 GDN oracle (numpy, BLAS threads) stepping a bounded sample of
    the same workload: 4 sequences x 32 heads through the tokens, repeated up
    to about target_s seconds, scaled to the batch."""
    from oracle import gdn as ogdn
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    nseq, tk = 4, w.steps
    sl = slice(0, nseq)
    t0 = time.perf_counter()
    passes, nsteps = 0, tk.steps
    while passes == 0 or (time.perf_counter() - t0 < target_s and passes < 20):
        ogdn.conventional(w.S0[sl], tk.q[:, sl], tk.k[:, sl], tk.v[:, sl], tk.g[:, sl], tk.beta[:, sl])
        passes += 1
    el = time.perf_counter() - t0
    step_s = el / (passes * nsteps) * w.shape.batch / nseq
    sh = w.shape
    host_bytes = 2 * sh.batch * sh.nv * sh.dv * sh.dk * 8        # the fp64 state read and written per step
    return {"value": round(host_bytes / step_s / 1e9, 3), "unit": "GB/s",
            "bytes_counted": "fp64 state read + written per step (2 x 4 MiB per sequence)",
            "gpu_bytes_rate_gbs": round(gpu_bytes_per_step / step_s / 1e9, 4),
            "us_per_step": round(step_s * 1e6, 1), "cores": threads, "kind": "oracle",
            "sample": f"{nseq} sequences x 32 heads x {nsteps} tokens, {passes} pass(es), {el:.1f} s "
                      f"(fp64 gated delta rule, numpy), scaled to {w.shape.batch} sequences",
            "host_cpu": _cpu_model()}


def cpu_baseline(work, gpu_bytes_per_step, target_s):
    """The fp64 oracle on a bounded sample of the same workload.

    The oracle steps every sequence (all heads) of the workload through its 64
    decode tokens, repeated until about `target_s` seconds have passed.  value:
    host GB/s of the fp64 state it reads and writes per step (2 x 8 MiB per
    sequence); us_per_step is the figure to compare with the GPU's step time,
    and gpu_bytes_rate_gbs the GPU step's algorithmic bytes over the oracle's
    step time (the step-rate ratio in GB/s)."""
    from oracle import oracle as orc
    o = orc.default()
    cores = o.num_threads()
    batch = work.shape.batch
    seqs = np.arange(batch)
    nsteps = work.steps.steps
    t0 = time.perf_counter()
    elapsed, passes = 0.0, 0
    while passes == 0 or (time.perf_counter() - t0 < target_s and passes < 50):
        elapsed += orc.time_decode(work, seqs, nsteps)
        passes += 1
    step_s = elapsed / (passes * nsteps)
    # one thread, 8 sequences (all heads), scaled to the whole batch
    few = np.arange(min(8, batch))
    one_s = orc.time_decode(work, few, nsteps, threads=1) / nsteps * batch / len(few)
    sh = work.shape
    host_bytes = 2 * batch * sh.nheads * sh.headdim * sh.dstate * 8   # the fp64 state read and written per step
    return {
        "value": round(host_bytes / step_s / 1e9, 3),
        "unit": "GB/s",
        "bytes_counted": "fp64 state read + written per step (2 x 8 MiB per sequence)",
        "us_per_step": round(step_s * 1e6, 1),
        "gpu_bytes_rate_gbs": round(gpu_bytes_per_step / step_s / 1e9, 4),
        "cores": cores,
        "kind": "oracle",
        "sample": f"all {batch} sequences x 128 heads x {nsteps} decode tokens of the same workload, "
                  f"{passes} pass(es), {elapsed:.1f} s inside the oracle (fp64 conventional recurrence, "
                  f"OpenMP over sequence/head pairs)",
        "cores_available": orc.available_cores(),
        "single_thread": {"us_per_step": round(one_s * 1e6, 1),
                          "sample": f"{len(few)} sequences x 128 heads x {nsteps} tokens on 1 thread, "
                                    f"scaled to {batch} sequences"},
        "host_cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _device():
    import torch
    return torch, torch.device("cuda", 0)


def _verify_point(T, batch=512, L=16, rounds=64, seed=1003, snapshots=True):
    """One speculative-verification workload: T drafts per round, accepted ~
    U{0..T}, initial fill U{0..L-1}.  Replay: verify_drafts + commit (pointer
    move), and the same rounds with the commit fused into the next
    verification.  Baseline: the conventional kernel writing one FP32 snapshot
    per draft (T + 1 slots per sequence) + slot-select commit.  Same inputs and
    acceptance for both."""
    torch, dev = _device()
    from mamba_state_replay_amd import binding as rb
    from mamba_state_replay_amd import staging, synth, traffic
    shape = synth.LayerShape(batch=batch, nheads=128, headdim=64, dstate=128, ngroups=8, window=L,
                             max_drafts=T)
    work = synth.verify_workload(shape, rounds, T, seed=seed)
    cfg = staging.config(shape)
    st = staging.replay_state(cfg, work, dev)
    p = staging.params(work, dev)
    toks = staging.TokenStream(work.steps, dev, T=T)
    acc = torch.from_numpy(work.extra["accepted"]).to(dev)
    y = torch.empty((batch, T, 128, 64), device=dev)
    sz = traffic.sizes(128, 64, 128, 8, 2, None)
    acc_np = work.extra["accepted"]

    def schedule(n, passes):
        """Bytes per round of `passes` consecutive passes over the rounds, from fill n."""
        out = []
        for _ in range(passes):
            for r in range(rounds):
                fold = n >= L
                out.append(traffic.verify_bytes(sz, n, fold, T))
                n = np.where(fold, 0, n) + acc_np[r]
        return out, n

    def replay_round(r):
        rb.replayssm_verify_drafts(cfg, st, p, toks.call(r), y)
        rb.replayssm_commit(cfg, st, acc[r], T)
    for r in range(8):                       # warm-up on a throw-away copy of the state
        replay_round(r)
    st = staging.replay_state(cfg, work, dev)
    # pass 1: eager launches (per-round events); passes 2 and 3: the same rounds
    # captured in one HIP graph, a warm replay and a timed one
    rbytes, n_end = schedule(work.n0.astype(np.int64).copy(), 3)
    ms, per = timed_launches(replay_round, rounds, torch)
    gms = graph_time(replay_round, rounds, torch)
    meta = st.meta.cpu().numpy()
    assert np.all(meta[:, :, 1] == n_end[:, None]) and int(st.status.cpu()[0]) == 0
    replay_us = ms * 1e3 / rounds
    replay_graph_us = gms * 1e3 / rounds
    eager_bytes = float(np.mean(rbytes[:rounds]))
    graph_bytes = float(np.mean(rbytes[2 * rounds:]))

    # the same rounds with the commit fused into the next verification
    st = staging.replay_state(cfg, work, dev)

    def fused_round(r, first_pass=True):
        if r == 0 and first_pass:
            rb.replayssm_verify_drafts(cfg, st, p, toks.call(r), y)
        else:
            rb.replayssm_commit_verify(cfg, st, p, acc[(r - 1) % rounds], T, toks.call(r), y)
    fms, fper = timed_launches(fused_round, rounds, torch)
    fgms = graph_time(lambda r: fused_round(r, first_pass=False), rounds, torch)
    rb.replayssm_commit(cfg, st, acc[rounds - 1], T)
    meta = st.meta.cpu().numpy()
    assert np.all(meta[:, :, 1] == n_end[:, None]) and int(st.status.cpu()[0]) == 0
    fused_us = fms * 1e3 / rounds
    fused_graph_us = fgms * 1e3 / rounds
    ring = batch * 128 * cfg.cap * (64 * 2 + 4) + batch * 8 * cfg.cap * 128 * 2
    del st
    torch.cuda.empty_cache()
    out = {
        "T": T,
        "replay": {"us_per_round": round(replay_graph_us, 2),
                   "gbs": round(graph_bytes / (replay_graph_us * 1e-6) / 1e9, 1),
                   "eager_us_per_round": round(replay_us, 2),
                   "eager_gbs": round(eager_bytes / (replay_us * 1e-6) / 1e9, 1),
                   "algorithmic_bytes_per_round": int(graph_bytes),
                   "state_bytes": batch * sz.S + ring},
        "replay_fused_commit": {"us_per_round": round(fused_graph_us, 2),
                                "gbs": round(graph_bytes / (fused_graph_us * 1e-6) / 1e9, 1),
                                "eager_us_per_round": round(fused_us, 2),
                                "launches_per_round": 1},
        "mean_accepted": float(work.extra["accepted"].mean()),
    }
    if snapshots:
        states = staging.conventional_states(cfg, work.h0, T + 1, dev)
        slot = torch.zeros(batch, dtype=torch.int32, device=dev)

        def snapshot_round(r):
            rb.conventional_state_update(cfg, states, p, toks.call(r), y, slot=slot)
            rb.conventional_commit(cfg, slot, T + 1, acc[r], T)
        for r in range(8):
            snapshot_round(r)
        slot.zero_()
        cms, cper = timed_launches(snapshot_round, rounds, torch)
        cgms = graph_time(snapshot_round, rounds, torch)
        snap_eager_us = cms * 1e3 / rounds
        snap_us = cgms * 1e3 / rounds
        sbytes = traffic.snapshot_verify_bytes(sz, batch, T)
        del states
        torch.cuda.empty_cache()
        out["snapshot_baseline"] = {"us_per_round": round(snap_us, 2),
                                    "gbs": round(sbytes / (snap_us * 1e-6) / 1e9, 1),
                                    "eager_us_per_round": round(snap_eager_us, 2),
                                    "algorithmic_bytes_per_round": sbytes,
                                    "state_bytes": (T + 1) * batch * sz.S}
        out["speedup"] = round(snap_us / replay_graph_us, 3)
        out["speedup_fused"] = round(snap_us / fused_graph_us, 3)
        out["timing"] = ("us_per_round: the rounds captured in one HIP graph, one replay timed after a warm "
                         "replay; eager_*: one Python call per launch")
    return out


def bench_verify(args):
    """Speculative verification at batch 512, T = 3, 64 rounds."""
    pt = _verify_point(3)
    out = {
        "metric": "speculative verify round us (T=3 drafts, batch 512) + achieved HBM GB/s",
        "config": {"workload": "Nemotron-3-style Mamba-2 layer, batch 512, T=3 drafts per round, accepted "
                               "U{0..3}, 64 rounds, L=16, initial fill U{0..15}", "batch": 512, "T": 3},
        **{k: v for k, v in pt.items() if k != "T"},
        "data": "synthetic", "n_gpus": 1,
    }
    print(json.dumps(out), flush=True)


def bench_verify_sweep(args):
    """Speculative verification at batch 512, L = 16, for T in {1, 2, 3, 4, 8}
    drafts per round (32 rounds each), replay against FP32 snapshots."""
    pts = []
    for T in (1, 2, 3, 4, 8):
        pts.append(_verify_point(T, rounds=32))
        print(json.dumps({"progress": f"T={T} done", "replay_us": pts[-1]["replay"]["us_per_round"]}), flush=True)
    print(json.dumps({"metric": "speculative verify round us vs drafts per round (batch 512, L=16)",
                      "config": {"workload": "Nemotron-3-style Mamba-2 layer, batch 512, L=16, accepted U{0..T}, "
                                             "32 rounds per point, initial fill U{0..15}"},
                      "points": pts, "data": "synthetic", "n_gpus": 1}), flush=True)


def bench_sweep(args):
    """Batch x window grid of the same layer, steady state (L committed records
    at start).  Per point: replay amortised us per step, its non-flush and
    flush launches, and the conventional step.  Where one copy of the FP32 state
    would fit the 256 MB Infinity Cache (batch <= 64), R independent replicas of
    the whole layer state (checkpoint, ring, pointers; conventional states) are
    allocated so that R copies exceed 768 MiB, and consecutive launches rotate
    through them: every launch then streams its state from HBM.  Each replica
    runs a whole number of windows inside the timed region."""
    torch, dev = _device()
    from mamba_state_replay_amd import binding as rb
    from mamba_state_replay_amd import staging, synth, traffic
    ntok = 32
    rows = []
    sz = traffic.sizes(128, 64, 128, 8, 2, None)
    for batch in (1, 16, 64, 256, 512):
        state = batch * sz.S
        R = 1 if state > 256 * 2 ** 20 else -(-(768 * 2 ** 20) // state)
        for L in (4, 8, 16, 32):
            steps = 128 if R == 1 else R * L * -(-128 // (R * L))
            shape = synth.LayerShape(batch=batch, nheads=128, headdim=64, dstate=128, ngroups=8, window=L)
            work = synth.decode_workload(shape, ntok, seed=1002, n0=L)
            cfg = staging.config(shape)
            sts = [staging.replay_state(cfg, work, dev) for _ in range(R)]
            p = staging.params(work, dev)
            toks = staging.TokenStream(work.steps, dev)
            y = torch.empty((batch, 1, 128, 64), device=dev)
            for j in range(2 * L):
                for st in sts:
                    rb.replayssm_decode_step(cfg, st, p, toks.call(j % ntok), y)
            sched, _ = traffic.decode_schedule(work.n0, L, 2 * L + steps // R)
            sched = [sched[2 * L + i // R] for i in range(steps)]
            rbytes = sum(traffic.decode_step_bytes(sz, n, f) for n, f in sched)
            rstep = lambda i: rb.replayssm_decode_step(cfg, sts[i % R], p, toks.call((2 * L + i // R) % ntok), y)
            ms, per = timed_launches(rstep, steps, torch)
            gms = graph_time(rstep, steps, torch)      # each replica runs whole windows: same phase
            folds = np.array([f.any() for _, f in sched])
            per = np.array(per)
            del sts
            torch.cuda.empty_cache()
            states = [staging.conventional_states(cfg, work.h0, 1, dev) for _ in range(R)]
            for i in range(4):
                rb.conventional_state_update(cfg, states[i % R], p, toks.call(i % ntok), y)
            cstep = lambda i: rb.conventional_state_update(cfg, states[i % R], p, toks.call((i // R) % ntok), y)
            cms, cper = timed_launches(cstep, steps, torch)
            cgms = graph_time(cstep, steps, torch)
            cbytes = traffic.conventional_step_bytes(sz, batch)
            r_us, c_us = ms * 1e3 / steps, cms * 1e3 / steps
            rg_us, cg_us = gms * 1e3 / steps, cgms * 1e3 / steps
            rows.append({"batch": batch, "L": L, "replay_us": round(r_us, 2),
                         "replay_nonflush_us": round(float(per[~folds].mean()) * 1e3, 2),
                         "replay_flush_us": round(float(per[folds].mean()) * 1e3, 2) if folds.any() else None,
                         "replay_gbs": round(rbytes / steps / (r_us * 1e-6) / 1e9, 1),
                         "conventional_us": round(c_us, 2),
                         "conventional_gbs": round(cbytes / (c_us * 1e-6) / 1e9, 1),
                         "speedup": round(c_us / r_us, 3),
                         "replay_graph_us": round(rg_us, 2), "conventional_graph_us": round(cg_us, 2),
                         "speedup_graph": round(cg_us / rg_us, 3),
                         "replay_graph_gbs": round(rbytes / steps / (rg_us * 1e-6) / 1e9, 1),
                         "state_replicas": R, "steps": steps})
            del states
            torch.cuda.empty_cache()
        print(json.dumps({"progress": f"batch {batch} done"}), flush=True)
    print(json.dumps({"metric": "decode-step us, replay vs conventional, batch x L sweep",
                      "config": {"workload": "Nemotron-3-style Mamba-2 layer, >= 128 decode steps per point, "
                                             "steady state; batch <= 64 rotates state replicas past the "
                                             "Infinity Cache"},
                      "points": rows, "data": "synthetic", "n_gpus": 1}), flush=True)


def bench_dual(args):
    """Dual precision: FP32 checkpoint with no copy, a bf16 copy, an e4m3 copy
    (one scale per head), an MXFP4 copy (E2M1 codes) or an MXFP8 copy (e4m3
    codes), the MX copies with one E8M0 scale per 32 columns; and an FP16
    checkpoint written with stochastic rounding (a new seed every call), read
    directly or through an MXFP4 copy.  Throughput: batch 256, L = 16, 4096
    decode steps (token inputs cycle through 64 seeded steps).  The accuracy of
    the modes is tested on the GPU (tests/test_gpu_dual.py,
    tests/test_gpu_f16ckpt.py), not part of this timing."""
    res = dual_measure(4096)
    print(json.dumps({"metric": "dual-precision decode: us per step and HBM GB/s (batch 256, L=16, 4096 steps)",
                      "config": {"workload": "Nemotron-3-style Mamba-2 layer, batch 256, L=16, 4096 decode steps"},
                      "modes": res, "data": "synthetic", "n_gpus": 1}), flush=True)


def dual_measure(steps):
    """Decode with each read copy and with the FP16 checkpoint (batch 256,
    L = 16, `steps` steps, a whole number of windows): per mode the graph-timed
    step, its algorithmic GB/s, and the mean non-flush and flush launch."""
    torch, dev = _device()
    from mamba_state_replay_amd import binding as rb
    from mamba_state_replay_amd import staging, synth, traffic
    L = 16
    assert steps % L == 0
    res = {}
    shape = synth.LayerShape(batch=256, nheads=128, headdim=64, dstate=128, ngroups=8, window=L)
    work = synth.decode_workload(shape, 64, seed=1004, n0=L)
    modes = [("f32", m) for m in (None, "bf16", "e4m3", "mxfp4", "mxfp8")] + [("f16", None), ("f16", "mxfp4")]
    for ck, mode in modes:
        cfg = staging.config(shape, read_copy=mode, ckpt_dtype=ck)
        st = staging.replay_state(cfg, work, dev)
        p = staging.params(work, dev)
        toks = staging.TokenStream(work.steps, dev)
        y = torch.empty((256, 1, 128, 64), device=dev)
        rb.replayssm_flush(cfg, st, p, rb.RSSM_FLUSH_FORCE_CAST)
        n0 = np.zeros(256, np.int64)
        sched, _ = traffic.decode_schedule(n0, L, steps)
        sz = traffic.sizes(128, 64, 128, 8, 2, mode, ckpt_bytes=4 if ck == "f32" else 2)
        tot = sum(traffic.decode_step_bytes(sz, n, f) for n, f in sched)

        def dstep(i):
            p.sr_seed = i + 1                   # the FP16 checkpoint's rounding seed (unused for FP32)
            rb.replayssm_decode_step(cfg, st, p, toks.call(i % 64), y)
        ms, per = timed_launches(dstep, steps, torch)
        gms = graph_time(dstep, steps, torch)          # whole windows: the replays start in the same phase
        per = np.array(per)
        folds = np.array([f.any() for _, f in sched])
        key = (mode or "fp32") if ck == "f32" else "f16 checkpoint" + (f" + {mode}" if mode else "")
        res[key] = {"us_per_step": round(gms * 1e3 / steps, 2),
                               "gbs": round(tot / (gms * 1e-3) / 1e9, 1),
                               "eager_us_per_step": round(ms * 1e3 / steps, 2),
                               "nonflush_launch_us": round(float(per[~folds].mean()) * 1e3, 2),
                               "flush_launch_us": round(float(per[folds].mean()) * 1e3, 2)}
        del st
        torch.cuda.empty_cache()
    return res


PROFILE_CMDS = {
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- "
             "python -u bench.py --no-cpu --no-conventional --no-extras --steps 16 --warmup 16",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- "
             "python -u bench.py --no-cpu --no-conventional --no-extras --steps 16 --warmup 16",
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof -o trace -- "
             "python -u bench.py --no-cpu --no-extras --steps 32 --warmup 16",
}


CONFIG_SUMMARY = ROOT / "profiles" / "bench_configs_verify_sweep_dual.md"


def summarize_configs(logs):
    """Write the tables of the verify / verify_sweep / sweep / dual bench lines
    (the last JSON line of each log, in any order) to profiles/."""
    lines = {}
    for path in logs:
        for line in reversed(Path(path).read_text().splitlines()):
            if line.startswith("{") and '"metric"' in line:
                d = json.loads(line)
                key = ("verify_sweep" if "drafts per round" in d["metric"] else
                       "verify" if "verify" in d["metric"] else
                       "sweep" if "sweep" in d["metric"] else "dual")
                lines[key] = d
                break
    md = ["# Bench configurations beyond the headline decode step (one MI355X)", "",
          "Commands (from the repository root):", "", "```"]
    md += [f"python -u bench.py --config {k}" for k in ("verify", "verify_sweep", "sweep", "dual") if k in lines]
    md += ["```", "", "Per-step and per-round times are one replay of the steps captured in a HIP graph (after a "
           "warm replay), timed with HIP events on the launch stream; \"eager\" times have one Python call "
           "per launch and an event pair around each; launch times are those event pairs. GB/s are "
           "algorithmic bytes (mamba_state_replay_amd/traffic.py) over the time.", ""]
    if "verify" in lines:
        v = lines["verify"]
        md += ["## Speculative verification: batch 512, T = 3, accepted U{0..3}, 64 rounds, L = 16", "",
               "| | us per round | eager us per round | algorithmic GB/s | bytes per round | state + buffer bytes |",
               "|---|---|---|---|---|---|",
               f"| replay: verify_drafts + commit | {v['replay']['us_per_round']} | "
               f"{v['replay'].get('eager_us_per_round')} | {v['replay']['gbs']} | "
               f"{v['replay']['algorithmic_bytes_per_round']:,} | {v['replay']['state_bytes']:,} |",
               f"| replay: commit fused into the next verification | {v['replay_fused_commit']['us_per_round']} | "
               f"{v['replay_fused_commit'].get('eager_us_per_round')} | "
               f"{v['replay_fused_commit']['gbs']} | same | same |",
               f"| conventional with one FP32 snapshot per draft + slot commit | "
               f"{v['snapshot_baseline']['us_per_round']} | {v['snapshot_baseline'].get('eager_us_per_round')} | "
               f"{v['snapshot_baseline']['gbs']} | "
               f"{v['snapshot_baseline']['algorithmic_bytes_per_round']:,} | "
               f"{v['snapshot_baseline']['state_bytes']:,} |", "",
               f"Speed-up of a verification round: {v['speedup']}x (fused commit: {v['speedup_fused']}x).", ""]
    if "verify_sweep" in lines:
        md += ["## Verification vs drafts per round: batch 512, L = 16, accepted U{0..T}, 32 rounds per point", "",
               "| T | replay us/round | fused us/round | replay GB/s | snapshot us/round | snapshot GB/s | speed-up | "
               "replay state bytes | snapshot state bytes |", "|---|---|---|---|---|---|---|---|---|"]
        for pt in lines["verify_sweep"]["points"]:
            sb = pt["snapshot_baseline"]
            md.append(f"| {pt['T']} | {pt['replay']['us_per_round']} | {pt['replay_fused_commit']['us_per_round']} | "
                      f"{pt['replay']['gbs']} | {sb['us_per_round']} | {sb['gbs']} | {pt['speedup']} | "
                      f"{pt['replay']['state_bytes']:,} | {sb['state_bytes']:,} |")
        md.append("")
    if "sweep" in lines:
        md += ["## Batch x window sweep, steady state", "",
               "Eager: one Python call per launch, events around each launch. Graph: the same launches captured "
               "in one HIP graph, one replay timed (GPU time without the host's per-launch cost).", "",
               "| batch | L | replay us/step | non-flush launch us | flush launch us | conventional us/step | "
               "speed-up | replay GB/s | graph: replay us/step | graph: conventional us/step | graph: speed-up | "
               "graph: replay GB/s | state replicas rotated | steps |",
               "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for pt in lines["sweep"]["points"]:
            md.append(f"| {pt['batch']} | {pt['L']} | {pt['replay_us']} | {pt['replay_nonflush_us']} | "
                      f"{pt['replay_flush_us']} | {pt['conventional_us']} | {pt['speedup']} | {pt['replay_gbs']} | "
                      f"{pt.get('replay_graph_us')} | {pt.get('conventional_graph_us')} | {pt.get('speedup_graph')} | "
                      f"{pt.get('replay_graph_gbs')} | {pt['state_replicas']} | {pt['steps']} |")
        md += ["", "Where one copy of the FP32 state fits the 256 MB Infinity Cache (batch <= 64), launches rotate "
               "through enough independent replicas of the layer state to exceed 768 MiB, so every launch "
               "streams its state from HBM.", ""]
    if "dual" in lines:
        md += ["## Dual precision: batch 256, L = 16, 4096 decode steps", "",
               "| checkpoint / read copy | us per step | eager us per step | algorithmic GB/s | non-flush launch us | "
               "flush launch us |",
               "|---|---|---|---|---|---|"]
        for k, m in lines["dual"]["modes"].items():
            md.append(f"| {k} | {m['us_per_step']} | {m.get('eager_us_per_step')} | {m['gbs']} | "
                      f"{m['nonflush_launch_us']} | {m['flush_launch_us']} |")
        md.append("")
    CONFIG_SUMMARY.write_text("\n".join(md) + "\n")
    print(f"wrote {CONFIG_SUMMARY}")


GDN_PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/gprof -o trace -- "
             "python -u bench.py --config gdn --no-cpu --steps 32 --warmup 17",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/gpmc_fetch -o fetch -- "
             "python -u bench.py --config gdn --no-cpu --steps 16 --warmup 17",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/gpmc_write -o write -- "
             "python -u bench.py --config gdn --no-cpu --steps 16 --warmup 17",
}


def ingest_gdn_counters(fetch_dir, write_dir, trace_dir):
    """Summarise the GDN runs of GDN_PROFILE_CMDS into profiles/.

    The bench's eager decode launches are the replay-kernel dispatches warmup ..
    warmup + steps - 1 (in dispatch order); counters are scaled by what they
    read for the 1 GiB copy probe of the same run."""
    import csv
    from mamba_state_replay_amd import traffic

    def bench_line(d):
        log = Path(d).parent / (Path(d).name + ".log")
        for line in reversed(log.read_text().splitlines()):
            if line.startswith("{"):
                return json.loads(line)
        raise ValueError(f"no bench JSON line in {log}")

    def eager(rows, key, line):
        rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
        W, K = line["warmup"], line["steps"]
        return rows[W:W + K]

    def counters(d, name):
        rows = list(csv.DictReader(open(next(Path(d).glob("*counter_collection.csv")))))
        line = bench_line(d)
        rep = eager([r for r in rows if "gdn_replay_kernel" in r["Kernel_Name"] and r["Counter_Name"] == name],
                    name, line)
        cp = [float(r["Counter_Value"]) for r in rows
              if "probe_copy_kernel" in r["Kernel_Name"] and r["Counter_Name"] == name]
        return [float(r["Counter_Value"]) for r in rep], cp, line

    f_rep, f_cp, fl = counters(fetch_dir, "FETCH_SIZE")
    w_rep, w_cp, wl = counters(write_dir, "WRITE_SIZE")
    assert fl["kernel_source_hash"] == wl["kernel_source_hash"]
    gib_kib = (1 << 30) / 1024
    ff, wf = gib_kib / float(np.mean(f_cp)), gib_kib / float(np.mean(w_cp))
    fetch_b, write_b = float(np.mean(f_rep)) * ff * 1024, float(np.mean(w_rep)) * wf * 1024
    L, batch, W, K = fl["config"]["window"], fl["config"]["batch"], fl["warmup"], fl["steps"]
    sched, _ = traffic.decode_schedule(np.zeros(batch, np.int64), L, W + K)
    sz = traffic.gdn_sizes(GDN_LAYER["nv"], GDN_LAYER["nk"], GDN_LAYER["dk"], GDN_LAYER["dv"])
    alg = float(np.mean([traffic.decode_step_bytes(sz, n, f) for n, f in sched[W:W + K]]))
    out = {"kernel": "gdn_replay_kernel<128, bf16 inputs>", "batch": batch, "window": L, "dispatches": len(f_rep),
           "source_hash": fl["kernel_source_hash"],
           "fetch_kib_per_dispatch": round(float(np.mean(f_rep)), 1),
           "write_kib_per_dispatch": round(float(np.mean(w_rep)), 1),
           "fetch_scale": round(ff, 4), "write_scale": round(wf, 4),
           "bytes_per_launch": int(fetch_b + write_b), "algorithmic_bytes_per_launch": int(alg),
           "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 4),
           "commands": [GDN_PROFILE_CMDS["fetch"], GDN_PROFILE_CMDS["write"]]}
    (ROOT / "profiles" / "gdn_decode_batch512_L16_counters.json").write_text(json.dumps(out, indent=1) + "\n")

    trows = list(csv.DictReader(open(next(Path(trace_dir).glob("*kernel_trace.csv")))))
    tl = bench_line(trace_dir)
    dec = eager([r for r in trows if "gdn_replay_kernel" in r["Kernel_Name"]], None, tl)
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in dec]
    tsched, _ = traffic.decode_schedule(np.zeros(batch, np.int64), L, tl["warmup"] + tl["steps"])
    tsched = tsched[tl["warmup"]:tl["warmup"] + tl["steps"]]
    fl_d = [d for d, (_, f) in zip(dur, tsched) if f.any()]
    nf_d = [d for d, (_, f) in zip(dur, tsched) if not f.any()]
    stats = list(csv.DictReader(open(next(Path(trace_dir).glob("*kernel_stats.csv")))))
    md = ["# GDN layer decode, batch 512, L = 16 (32 value heads over 16 key heads, dk = dv = 128): "
          "kernel trace and HBM counters", "", "Kernel trace (one MI355X):", "", "```", GDN_PROFILE_CMDS["trace"],
          "```", "", "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "gdn_" not in r["Name"] and "probe_copy" not in r["Name"] and "commit" not in r["Name"]:
            continue
        name = r["Name"].replace("void ", "").replace("rssm::(anonymous namespace)::", "").split("(")[0]
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    md += ["", "The replay kernel's calls mix decode (T = 1) and verify (T = 3) launches. Its "
           f"{len(dur)} eager decode launches of the timed region (dispatches {tl['warmup']} .. "
           f"{tl['warmup'] + tl['steps'] - 1}): average {np.mean(dur):.2f} us, non-flush {np.mean(nf_d):.2f} us, "
           f"flush {np.mean(fl_d) if fl_d else float('nan'):.2f} us (bench line of the same run: "
           f"{tl['roofline']['avg_launch_us']} us average).", "",
           "HBM counters (separate runs, one counter each; the eager decode launches):", "", "```",
           GDN_PROFILE_CMDS["fetch"], GDN_PROFILE_CMDS["write"], "```", "",
           "| | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |", "|---|---|---|",
           f"| gdn_replay_kernel (average of {len(f_rep)} decode dispatches) | {np.mean(f_rep):.1f} | "
           f"{np.mean(w_rep):.1f} |",
           f"| probe_copy_kernel, 1 GiB read + 1 GiB written | {np.mean(f_cp):.1f} | {np.mean(w_cp):.1f} |", "",
           f"Scale factors from the copy probe: FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {wf:.4f}.",
           f"GDN replay kernel: {fetch_b / 1e9:.4f} GB fetched + {write_b / 1e9:.4f} GB written = "
           f"{(fetch_b + write_b) / 1e9:.4f} GB per launch, against {alg / 1e9:.4f} GB algorithmic "
           f"(ratio {(fetch_b + write_b) / alg:.4f}).", f"Kernel source hash {fl['kernel_source_hash']}."]
    (ROOT / "profiles" / "gdn_decode_batch512_L16.md").write_text("\n".join(md) + "\n")
    print(json.dumps(out))


_SQ_SET = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_INSTS_VALU SQ_INSTS_SALU "
           "SQ_INSTS_LDS")
_MX_CMD = "python -u bench.py --read-copy mxfp4 --no-cpu --no-conventional --no-extras --steps 16 --warmup 16"
SQ_PROFILE_CMDS = {
    "fetch": f"rocprofv3 --pmc FETCH_SIZE -d gpurun_out/mx_fetch -o fetch -- {_MX_CMD}",
    "write": f"rocprofv3 --pmc WRITE_SIZE -d gpurun_out/mx_write -o write -- {_MX_CMD}",
    "sq": f"rocprofv3 --pmc {_SQ_SET} -d gpurun_out/mx_sq -o sq -- {_MX_CMD}",
    "sq_f32": f"rocprofv3 --pmc {_SQ_SET} -d gpurun_out/f32_sq -o sq -- "
              "python -u bench.py --no-cpu --no-conventional --no-extras --steps 16 --warmup 16",
}


def ingest_sq_counters():
    """Summarise the runs of SQ_PROFILE_CMDS: per-dispatch HBM bytes of the
    MXFP4 read-copy kernel (non-flush and flush dispatches apart, scaled by the
    copy probe of the same run) and per-wave SQ counters of that kernel, the
    FP32 kernel and the streaming read probe."""
    import collections
    import sqlite3
    import statistics

    def per_dispatch(d):
        db = sorted(Path(d).rglob("*.db"))[0]
        rows = sqlite3.connect(str(db)).execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection").fetchall()
        vals = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for did, kn, cn, v in rows:
            vals[did][cn] += v
            names[did] = kn
        return vals, names

    def ids(names, key):
        return [d for d in sorted(names) if key in names[d]]

    mx = "replay_kernel<64, 128, 256, unsigned short, 3, 4, 4, false>"
    f32 = "replay_kernel<64, 128, 256, unsigned short, 0, 1, 4, false>"
    f, fn = per_dispatch("gpurun_out/mx_fetch")
    w, wn = per_dispatch("gpurun_out/mx_write")
    fs = [f[d]["FETCH_SIZE"] for d in ids(fn, mx)]
    ws = [w[d]["WRITE_SIZE"] for d in ids(wn, mx)]
    med = statistics.median(fs)
    flush_idx = [i for i, v in enumerate(fs) if v > 3 * med]     # they read the FP32 checkpoint
    nonflush_idx = [i for i in range(len(fs)) if i not in set(flush_idx)]
    fscale = round(1048576.0 / statistics.median(f[d]["FETCH_SIZE"] for d in ids(fn, "probe_copy_kernel")), 4)
    wscale = round(1048576.0 / statistics.median(w[d]["WRITE_SIZE"] for d in ids(wn, "probe_copy_kernel")), 4)
    rows = []
    for label, idx in (("non-flush", nonflush_idx), ("flush", flush_idx)):
        fk = sum(fs[i] for i in idx) / len(idx)
        wk = sum(ws[i] for i in idx) / len(idx)
        rows.append(f"| {label} ({len(idx)} dispatches) | {fk:.1f} | {wk:.1f} | "
                    f"{(fk * fscale + wk * wscale) * 1024 / 1e9:.4f} |")

    cols = ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_INSTS_VALU",
            "SQ_INSTS_SALU", "SQ_INSTS_LDS"]
    sqrows = []
    for label, d, key, idx in (("MXFP4 copy, non-flush", "gpurun_out/mx_sq", mx, nonflush_idx),
                               ("MXFP4 copy, flush", "gpurun_out/mx_sq", mx, flush_idx),
                               ("FP32 checkpoint, all decode launches", "gpurun_out/f32_sq", f32, None),
                               ("streaming read probe (1 GiB)", "gpurun_out/f32_sq", "probe_read_kernel", None)):
        vals, names = per_dispatch(d)
        sel = ids(names, key)
        if idx is not None:                  # the same launch order as the HBM-counter runs
            sel = [sel[i] for i in idx if i < len(sel)]
        tot = collections.defaultdict(float)
        for i in sel:
            for k, v in vals[i].items():
                tot[k] += v
        per = {k: round(v / tot["SQ_WAVES"], 1) for k, v in tot.items() if k != "SQ_WAVES"}
        sqrows.append(f"| {label} ({len(sel)}) | " + " | ".join(str(per.get(c, "")) for c in cols) + " |")

    md = ["# Mamba-2 decode, batch 256, L = 16: HBM and SQ counters of the MXFP4 read-copy kernel "
          "(and the FP32 kernel's SQ counters)", "", "Commands (one MI355X; one counter set per run):", "", "```"]
    md += [SQ_PROFILE_CMDS[k] for k in ("fetch", "write", "sq", "sq_f32")]
    md += ["```", "",
           f"Kernel `{mx}` (sixth template argument: 4 heads per workgroup). Dispatches whose FETCH_SIZE "
           "exceeds three times the median are the flushing calls (they read the FP32 checkpoint and write it "
           "and the copy).",
           f"Scale factors from the copy probe in the same runs (1 GiB read + 1 GiB written): FETCH_SIZE x "
           f"{fscale}, WRITE_SIZE x {wscale}.", "",
           "| dispatches | FETCH_SIZE KiB per dispatch | WRITE_SIZE KiB per dispatch | scaled HBM GB per dispatch |",
           "|---|---|---|---|"] + rows
    md += ["", "The non-flush calls' algorithmic bytes at the steady state's average of 8 committed records are "
           "about 0.200 GB (codes, scale bytes, records, tokens, outputs; `mamba_state_replay_amd/traffic.py`).",
           "", "SQ counters, per wave (cycle counters in the counter's own units):", "",
           "| kernel (dispatches) | " + " | ".join(cols) + " |", "|---" * (len(cols) + 1) + "|"] + sqrows
    out = ROOT / "profiles" / "replay_decode_batch256_L16_sq_counters.md"
    out.write_text("\n".join(md) + "\n")
    print(f"wrote {out}")


def ingest_counters(fetch_dir, write_dir, trace_dir):
    """Turn the rocprofv3 CSVs of PROFILE_CMDS into profiles/ summaries.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read
    for the 1 GiB copy probe in the same run (its true traffic is 1 GiB read +
    1 GiB written), then averaged over the replay kernel's dispatches."""
    import csv
    from mamba_state_replay_amd import traffic

    def counters(d, name):
        rows = list(csv.DictReader(open(next(Path(d).glob("*counter_collection.csv")))))
        rep = [float(r["Counter_Value"]) for r in rows
               if "replay_kernel" in r["Kernel_Name"] and r["Counter_Name"] == name]
        cp = [float(r["Counter_Value"]) for r in rows
              if "probe_copy_kernel" in r["Kernel_Name"] and r["Counter_Name"] == name]
        return rep, cp

    def bench_line(d):
        log = Path(d).parent / (Path(d).name + ".log")
        for line in reversed(log.read_text().splitlines()):
            if line.startswith("{"):
                return json.loads(line)
        raise ValueError(f"no bench JSON line in {log}")

    f_rep, f_cp = counters(fetch_dir, "FETCH_SIZE")
    w_rep, w_cp = counters(write_dir, "WRITE_SIZE")
    line = bench_line(fetch_dir)
    assert bench_line(write_dir)["kernel_source_hash"] == line["kernel_source_hash"]
    gib_kib = (1 << 30) / 1024
    ff = gib_kib / float(np.mean(f_cp))
    wf = gib_kib / float(np.mean(w_cp))
    fetch_b = float(np.mean(f_rep)) * ff * 1024
    write_b = float(np.mean(w_rep)) * wf * 1024
    L, batch = line["config"]["window"], line["config"]["batch"]
    sched, _ = traffic.decode_schedule(np.full(batch, L), L, len(f_rep))
    sz = traffic.sizes(128, 64, 128, 8, 2, None)
    alg = float(np.mean([traffic.decode_step_bytes(sz, n, f) for n, f in sched]))
    out = {
        "kernel": "replay_kernel<64, 128, 256, bf16 inputs, FP32 checkpoint read>",
        "batch": batch, "window": L, "dispatches": len(f_rep),
        "source_hash": line["kernel_source_hash"],
        "fetch_kib_per_dispatch": round(float(np.mean(f_rep)), 1),
        "write_kib_per_dispatch": round(float(np.mean(w_rep)), 1),
        "copy_probe_fetch_kib": round(float(np.mean(f_cp)), 1),
        "copy_probe_write_kib": round(float(np.mean(w_cp)), 1),
        "fetch_scale": round(ff, 4), "write_scale": round(wf, 4),
        "bytes_per_launch": int(fetch_b + write_b),
        "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
        "algorithmic_bytes_per_launch": int(alg),
        "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 4),
        "commands": [PROFILE_CMDS["fetch"], PROFILE_CMDS["write"]],
    }
    COUNTERS.write_text(json.dumps(out, indent=1) + "\n")

    rows = list(csv.DictReader(open(next(Path(trace_dir).glob("*kernel_stats.csv")))))
    md = ["# replay decode, batch 256, L = 16 (Nemotron-3-style Mamba-2 layer): kernel trace and HBM counters", "",
          "Kernel trace (one MI355X):", "", "```", PROFILE_CMDS["trace"], "```", "",
          "| kernel | calls | average us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        if "rssm::" not in r["Name"]:
            continue
        name = r["Name"].replace("void ", "").replace("rssm::(anonymous namespace)::", "").split("(")[0]
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    md += ["", "Template arguments: `<headdim, dstate, threads, input type (unsigned short = bf16 bits), "
           "read mode (0 = FP32 checkpoint), heads per workgroup>`. The replay average mixes non-flush and flush launches "
           "(one in 16 flushes); min is a non-flush launch, max a flush launch.", "",
           "HBM counters (separate runs, one counter each):", "", "```", PROFILE_CMDS["fetch"],
           PROFILE_CMDS["write"], "```", "",
           f"| | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |", "|---|---|---|",
           f"| replay_kernel (average of {len(f_rep)} dispatches) | {np.mean(f_rep):.1f} | {np.mean(w_rep):.1f} |",
           f"| probe_copy_kernel, 1 GiB read + 1 GiB written | {np.mean(f_cp):.1f} | {np.mean(w_cp):.1f} |", "",
           f"Scale factors from the copy probe: FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {wf:.4f}.",
           f"Replay kernel: {fetch_b / 1e9:.4f} GB fetched + {write_b / 1e9:.4f} GB written = "
           f"{(fetch_b + write_b) / 1e9:.4f} GB per launch, against {alg / 1e9:.4f} GB algorithmic "
           f"(ratio {(fetch_b + write_b) / alg:.4f}).",
           f"Kernel source hash {line['kernel_source_hash']}."]
    (ROOT / "profiles" / "replay_decode_batch256_L16.md").write_text("\n".join(md) + "\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
