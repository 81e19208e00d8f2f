#!/usr/bin/env python3
"""Throughput of one data-parallel rank's ZeRO step on its 1/N shard.

Default workload: the Llama-3-8B-shaped parameter list (psi = 8,030,261,248)
at N = 8, rank 0's shard of S = 1,003,782,656 parameters, fp16 contributions
~N(0, 1e-3) x 65536, AdamW lr 3e-4, wd 0.1, global clip at 1.0 (the other
seven ranks' squared norm stood in by a host scalar).

A step is one pass of the whole path: zero_reduce_check (reduce N fp16 rows,
unscale, overflow flag, exact squared norm, clip / skip decision) then
zero_adam_apply (AdamW on fp32 master, m, v and the fp16 slot write); this is
exactly what zero_reduce_adam_step enqueues.  Inputs are resident in HBM when
the timed region starts; every timed step is applied (no skip).

Prints one JSON line.  Fields beyond the common ones:
  roofline      the dominant kernel's algorithmic bytes per step over the
                HIP-event duration of its dispatches in a step (a long grid
                goes out as several consecutive dispatches), against the
                8 TB/s HBM peak; `traffic` is the counter-measured HBM bytes of
                the same dispatches
  kernels       the same figures for both kernels
  cpu_baseline  the CPU oracle timed on bounded windows of the same shard, in
                one process and in one process per host core (at most 16)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ("zero_sharded_optimizer_rank_amd/csrc/zero_kernels.hip",
                  "zero_sharded_optimizer_rank_amd/csrc/zero_units.hip",
                  "zero_sharded_optimizer_rank_amd/csrc/zero_noalloc.hip",
                  "zero_sharded_optimizer_rank_amd/csrc/zero_device.h",
                  "zero_sharded_optimizer_rank_amd/csrc/zero_internal.h")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def bytes_per_param(n: int):
    """Algorithmic bytes per shard element of each kernel on an applied step."""
    k1 = 2 * n + 4   # read N 16-bit contributions, write fp32 g
    k2 = 16 + 14     # read g, master, m, v; write master, m, v and the 16-bit slot
    return k1, k2


def traffic_for(workload: str, kernel: str):
    """Counter-derived HBM bytes of one step's dispatches of `kernel`, if
    recorded for the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_step")


def _oracle_inputs(w, begin: int, n: int):
    import oracle
    from oracle import run as orun

    p = orun.workload_plan(w)
    c = orun.shard_contrib(w, p, 0, 1, w.loss_scale0, begin, n)
    pm, m, v, h = orun.initial_state(w, p, 0, begin, n)
    other_sq = w.other_sq(p.real(0)) if w.other_ranks_from_config else 0.0
    return c, pm, m, v, h, other_sq


def _oracle_steps(w, inputs, reps: int = 0, seconds: float = 0.0):
    """Run the oracle's whole step on one window again and again, carrying the
    state: `reps` times, or until `seconds` have passed (at least twice).
    Returns (steps, elapsed seconds)."""
    import oracle

    c, pm, m, v, h, other_sq = inputs
    step_fn = oracle.shard_step_bf16 if w.dtype == "bf16" else oracle.shard_step
    done, t_applied, t0 = 0, 0, time.perf_counter()
    while True:
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, t_applied + 1,
                                 w.world_size, w.loss_scale0)
        out = step_fn(c, pm, m, v, h, sc, w.max_grad_norm, other_sq=other_sq)
        pm, m, v, h = out.p, out.m, out.v, out.h
        t_applied += 0 if out.fin.skip else 1
        done += 1
        el = time.perf_counter() - t0
        if (reps and done >= reps) or (not reps and done >= 2 and el >= seconds):
            return done, el


_BARRIER = None


def _pool_init(barrier):
    global _BARRIER
    _BARRIER = barrier


def _oracle_worker(args):
    """One process of the parallel baseline: its own window of the shard,
    generated before the common start, then `reps` oracle steps."""
    w, begin, n, reps = args
    inputs = _oracle_inputs(w, begin, n)
    _BARRIER.wait()
    t0 = time.time()
    done, _ = _oracle_steps(w, inputs, reps=reps)
    return n * done, t0, time.time()


def cpu_baseline(w, seconds: float, procs: int):
    """The oracle as it is, on rank 0's shard, timed on the host's cores:
    first one process on the first 2^25 elements for about `seconds`, then
    `procs` processes at once, each on its own 2^23-element window, for about
    as long.  Input generation is outside the timing.  The workers are fresh
    interpreters (spawned: the seeded generator's OpenMP runtime does not
    survive a fork), started before anything touches the GPU."""
    import multiprocessing as mp

    from oracle import run as orun

    shard = orun.workload_plan(w).shard
    n1 = min(1 << 25, shard)
    steps1, el1 = _oracle_steps(w, _oracle_inputs(w, 0, n1), seconds=seconds)
    rate1 = n1 * steps1 / el1
    out = {"unit": "params/s", "kind": "oracle",
           "single_process": {"value": rate1, "cores": 1,
                              "sample": f"{w.name} rank 0 shard elements [0, {n1}) x "
                                        f"{w.world_size} contributions, {steps1} oracle steps "
                                        f"(numpy, one process), {el1:.1f} s"}}
    nw = min(1 << 23, max(1, shard // max(procs, 1)))
    procs = min(procs, max(1, shard // nw))
    if procs <= 1:
        out.update(value=rate1, cores=1, sample=out["single_process"]["sample"])
        return out
    reps = max(2, int(seconds * rate1 / nw))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(procs)
    with ctx.Pool(procs, initializer=_pool_init, initargs=(barrier,)) as pool:
        res = pool.map(_oracle_worker, [(w, k * nw, nw, reps) for k in range(procs)])
    total = sum(r[0] for r in res)
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    out.update(value=total / wall, cores=procs,
               sample=f"{w.name} rank 0 shard, {procs} processes each on its own {nw}-element "
                      f"window x {w.world_size} contributions, {reps} oracle steps each "
                      f"(numpy, one thread per process), {wall:.1f} s wall")
    return out


def calibration_copy(nbytes: float, stream):
    """Time a one-shot copy of known size (measurement-only library): the
    ceiling a streaming kernel reaches on this part, and the known-size kernel
    the counter passes are scaled by.  The caller frees its buffers first."""
    if nbytes <= 0:
        return None
    import ctypes
    import torch
    from zero_sharded_optimizer_rank_amd.build import CALIB_LIB
    cl = ctypes.CDLL(CALIB_LIB)
    cl.zero_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p]
    nb = int(nbytes) // 16 * 16
    torch.cuda.empty_cache()
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    best = None
    for threads in (64, 256):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for rep in range(4):
            if rep == 1:
                e0.record(stream)
            rc = cl.zero_calib_copy(src.data_ptr(), dst.data_ptr(), nb, threads,
                                    stream.cuda_stream)
            assert rc == 0
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = 2 * nb * 3 / (e0.elapsed_time(e1) * 1e6)
        best = gbps if best is None else max(best, gbps)
    return {"copy_gbps": best, "bytes": nb}


# ---------------------------------------------------------------------------
# rocprofv3 summaries for profiles/: kernel durations from a --kernel-trace
# --stats run of this script, HBM bytes from two --pmc runs (FETCH_SIZE, then
# WRITE_SIZE), each scaled by what the same counter reads for the calibration
# copy of known size in the same run.

PROF_KERNELS = ("k12u_reduce_adam", "k12_reduce_adam_bf16", "k12_reduce_adam", "k1u_reduce_check",
                "k2u_adam", "k1_reduce_check_bf16", "k2_adam_bf16", "kt_tree_finalize_bf16",
                "k1_reduce_check", "kf_reduce_finalize", "k2_adam", "k_store_table", "calib_copy")


def _prof_short(name: str):
    for k in PROF_KERNELS:
        if k + "(" in name or name.endswith(k) or ("::" + k) in name:
            return k
    return None


def _prof_file(pattern: str, d: str) -> str:
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not f:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return f[0]


def _json_line(path: str) -> dict:
    with open(path) as f:
        lines = [ln for ln in f if ln.startswith("{")]
    if not lines:
        raise ValueError(f"no JSON line in {path}")
    return json.loads(lines[-1])


def summarize_rocprof(label: str, bench_args: str, pmc_args: str, out: str = "gpurun_out",
                      prof: str = ""):
    """Write profiles/<kernels>_<label>_{kernel_stats,hbm_traffic}.md and
    profiles/traffic_<label>.json (or into `prof`) from the rocprofv3 outputs
    that the commands written into those files leave under `out`."""
    import csv

    kt_dir = os.path.join(out, f"prof_kt_{label}")
    kt_log = os.path.join(out, f"bench_kt_{label}.log")
    j = _json_line(kt_log)
    S, N = int(j["config"]["shard"]), int(j["config"]["world_size_simulated"])
    one_pass = "single pass" in j["metric"]
    desc = j["config"]["workload"]

    def algo(k):
        if k.startswith("k12"):
            return (2 * N + 26) * S
        if k.startswith("k1"):
            return (2 * N + 4) * S
        if k.startswith("k2"):
            return 30 * S
        return None

    # A long grid goes out as several dispatches of one kernel per step, so
    # every figure below is per step: the sum over that kernel's dispatches,
    # divided by the number of steps (one finalize dispatch per step).
    stats = {}
    for r in csv.DictReader(open(_prof_file("*kernel_stats.csv", kt_dir))):
        k = _prof_short(r["Name"])
        if k is None:
            continue
        calls, avg = int(r["Calls"]), float(r["AverageNs"]) / 1e3
        v = stats.setdefault(k, dict(calls=0, total=0.0, mn=float("inf"), mx=0.0))
        v["calls"] += calls
        v["total"] += calls * avg
        v["mn"] = min(v["mn"], float(r["MinNs"]) / 1e3)
        v["mx"] = max(v["mx"], float(r["MaxNs"]) / 1e3)
    fin = "kt_tree_finalize_bf16" if "kt_tree_finalize_bf16" in stats else "kf_reduce_finalize"
    steps = stats[fin]["calls"] if fin in stats else 1

    def counters(cname):
        d = os.path.join(out, f"prof_{cname}_{label}")
        acc = {}
        for r in csv.DictReader(open(_prof_file("*counter_collection.csv", d))):
            if r["Counter_Name"] != cname:
                continue
            k = _prof_short(r["Kernel_Name"])
            if k is not None:
                acc.setdefault(k, []).append(float(r["Counter_Value"]))
        calib = float(_json_line(os.path.join(out, f"bench_{cname}_{label}.log"))
                      ["calibration_copy"]["bytes"])
        n_steps = len(acc.get("kt_tree_finalize_bf16", acc.get("kf_reduce_finalize", [0]))) or 1
        per_step = {k: sum(v) / n_steps for k, v in acc.items() if k != "calib_copy"}
        per_step["calib_copy"] = sum(acc["calib_copy"]) / len(acc["calib_copy"])
        per_disp = {k: len(v) / n_steps for k, v in acc.items()}
        return per_step, per_disp, calib

    fetch, disp_f, calib_f = counters("FETCH_SIZE")
    write, _, calib_w = counters("WRITE_SIZE")
    fs = calib_f / (fetch["calib_copy"] * 1024)
    ws = calib_w / (write["calib_copy"] * 1024)
    kh = kernel_hash()
    rec = {"kernel_hash": kh, "workload": label, "fetch_scale": fs, "write_scale": ws,
           "kernels": {}}
    for k in fetch:
        if k == "calib_copy":
            continue
        rb, wb = fetch[k] * 1024 * fs, write.get(k, 0.0) * 1024 * ws
        rec["kernels"][k] = {"read_bytes": rb, "write_bytes": wb, "bytes_per_step": rb + wb,
                             "dispatches_per_step": disp_f[k], "algorithmic_bytes": algo(k)}
    prof = prof or os.path.join(ROOT, "profiles")
    with open(os.path.join(prof, f"traffic_{label}.json"), "w") as f:
        json.dump(rec, f, indent=1)

    kt_cmd = (f"rocprofv3 --kernel-trace --stats -f csv -d {kt_dir} -o {label} -- "
              f"python3 bench.py {bench_args} --cpu-procs 1 > {kt_log}")
    pmc_cmds = [f"timeout -s KILL 300 rocprofv3 --pmc {c} -f csv -d {out}/prof_{c}_{label} "
                f"-o {label} -- python3 bench.py {pmc_args} > {out}/bench_{c}_{label}.log"
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
    sum_cmd = (f"python3 bench.py --summarize-rocprof {label} --bench-args \"{bench_args}\" "
               f"--pmc-args \"{pmc_args}\"")
    recipe = ("Commands (from the repository root on one MI355X, with TMPDIR=/tmp; the last "
              "one reads their output and writes this file):\n\n```\n" + kt_cmd + "\n"
              + "\n".join(pmc_cmds) + "\n" + sum_cmd + "\n```\n\n")
    prefix = "k12" if one_pass else "k1_k2"
    calib_kt = (j.get("calibration_copy") or {}).get("bytes")
    with open(os.path.join(prof, f"{prefix}_{label}_kernel_stats.md"), "w") as f:
        f.write(f"# Kernel durations: {desc}\n\n" + recipe +
                f"Kernel source hash (bench.py `kernel_hash`): `{kh}`.  {steps} steps traced "
                f"(one `{fin}` dispatch each).\n\n"
                "| kernel | dispatches | per step | avg per dispatch (us) | min (us) | max (us) "
                "| per step (us) | algorithmic bytes per step | GB/s |\n"
                "|---|---|---|---|---|---|---|---|---|\n")
        for k, v in sorted(stats.items(), key=lambda kv: -kv[1]["total"]):
            avg = v["total"] / v["calls"]
            if k == "calib_copy":
                a = 2 * calib_kt if calib_kt else None
                f.write(f"| {k} | {v['calls']} | - | {avg:.1f} | {v['mn']:.1f} | {v['mx']:.1f} "
                        f"| - | " + (f"{a / 1e9:.3f} GB per dispatch | {a / (avg * 1e3):.0f} |"
                                     if a else "- | - |") + "\n")
                continue
            per = v["total"] / steps
            a = algo(k)
            f.write(f"| {k} | {v['calls']} | {v['calls'] / steps:g} | {avg:.1f} | {v['mn']:.1f} "
                    f"| {v['mx']:.1f} | {per:.1f} | "
                    + (f"{a / 1e9:.3f} GB | {a / (per * 1e3):.0f} |" if a else "- | - |") + "\n")
        f.write("\nThe JSON line this traced run printed (HIP events on the launch stream, "
                "around all of a kernel's dispatches in a step):\n\n")
        for k, v in j["kernels"].items():
            f.write(f"- {k}: {v['ms'] * 1e3:.1f} us ({v['gbps']:.0f} GB/s)\n")
        f.write(f"- step {j['ms_per_step'] * 1e3:.1f} us, {j['value'] / 1e9:.2f} G params/s\n")
        f.write("\nOnly this library's kernels and the calibration copy (`calib_copy`, a one-shot "
                "copy of known size) are listed; torch's set-up kernels are left out.  "
                "A long grid is issued as several dispatches of one kernel, so `per step` is "
                "the dispatch count and the summed duration in one step; GB/s is the step's "
                "algorithmic bytes over that sum.  "
                "The reduce's deferred form (above N = 8) is listed "
                "under the one-chunk kernel's name (`k1_reduce_check`, `k1u_reduce_check`).  "
                "Algorithmic bytes: 2N + 4 per element for the reduce, 30 for the update, "
                "2N + 26 for the single pass.\n")
    with open(os.path.join(prof, f"{prefix}_{label}_hbm_traffic.md"), "w") as f:
        f.write(f"# HBM traffic per step: {desc}\n\n" + recipe +
                f"Kernel source hash: `{kh}`.  Counter values are KiB summed over a kernel's "
                "dispatches in one step (averaged over the steps).\n\n"
                f"Calibration: calib_copy moves exactly {calib_f:.0e} bytes each way per call. "
                f"FETCH_SIZE reads {fetch['calib_copy']:.1f} KiB for it (scale x{fs:.4f}); "
                f"WRITE_SIZE reads {write['calib_copy']:.1f} KiB (scale x{ws:.4f}).\n\n"
                "| kernel | dispatches per step | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes "
                "(scaled) | write bytes (scaled) | total | algorithmic | total / algorithmic |\n"
                "|---|---|---|---|---|---|---|---|---|\n")
        for k, v in rec["kernels"].items():
            a = v["algorithmic_bytes"]
            f.write(f"| {k} | {v['dispatches_per_step']:g} | {fetch[k]:.1f} | "
                    f"{write.get(k, 0):.1f} | "
                    f"{v['read_bytes'] / 1e9:.4f} GB | {v['write_bytes'] / 1e9:.4f} GB | "
                    f"{v['bytes_per_step'] / 1e9:.4f} GB | "
                    + (f"{a / 1e9:.4f} GB | {v['bytes_per_step'] / a:.4f} |" if a
                       else "- | - |") + "\n")
    print(f"wrote profiles for {label}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="processes of the parallel CPU oracle baseline (0: the CPUs this "
                         "process may use, at most 16; 1 under a GPU profiler, whose preloaded "
                         "library the worker processes would inherit)")
    ap.add_argument("--row-align", type=int, default=None,
                    help="contribution row stride alignment in elements (default: the runtime's)")
    ap.add_argument("--time-skip", action="store_true",
                    help="also time three steps forced to skip (kept out of the default run so "
                         "that a kernel trace of it holds applied steps only)")
    ap.add_argument("--offload", action="store_true",
                    help="time the offload form: reduce on the GPU, Adam on the host from "
                         "host-resident state, fp16 parameters back over PCIe")
    ap.add_argument("--threads", type=int, default=0,
                    help="host threads of the offload form (0: up to 8 of the CPUs this "
                         "process may use)")
    ap.add_argument("--one-stream", action="store_true",
                    help="offload form: both PCIe directions on one stream")
    ap.add_argument("--one-pass", action="store_true",
                    help="time zero_reduce_adam_step_1pass (steps without clipping: reduce and "
                         "update in one pass into a second state set, 2N + 26 bytes per element)")
    ap.add_argument("--in-place-slot", action="store_true",
                    help="--one-pass on a flat shard: write the live slot and call "
                         "zero_slot_restore after every step (timed with the step)")
    ap.add_argument("--no-clip", action="store_true",
                    help="turn the workload's gradient clipping off (a variant, named in the "
                         "config; needed for --one-pass on workloads that clip)")
    ap.add_argument("--calib-bytes", type=float, default=4e9,
                    help="bytes of the calibration copy timed next to the step (0: skip)")
    ap.add_argument("--summarize-rocprof", metavar="LABEL", default=None,
                    help="no GPU: write profiles/ summaries for LABEL from the rocprofv3 "
                         "output of the commands they list (with --bench-args, --pmc-args)")
    ap.add_argument("--bench-args", default="", help="--summarize-rocprof: the traced run's args")
    ap.add_argument("--pmc-args", default="", help="--summarize-rocprof: the counter runs' args")
    a = ap.parse_args()
    if a.summarize_rocprof:
        return summarize_rocprof(a.summarize_rocprof, a.bench_args, a.pmc_args)
    if a.gpus != 1:
        print("bench.py measures the shard step on one GPU only; --gpus must be 1 "
              "(the multi-GPU exchange around the step is not built)", file=sys.stderr)
        sys.exit(2)

    import synth

    w = synth.BY_NAME[a.workload]
    if a.no_clip:
        import dataclasses
        w = dataclasses.replace(w, max_grad_norm=0.0)
    # the CPU baseline starts worker processes: it runs before anything
    # touches the GPU
    cpu = None
    if (not a.no_cpu_baseline and w.units is None and not a.offload and not a.one_pass):
        cpu = cpu_baseline(w, a.cpu_seconds, a.cpu_procs or
                           max(1, min(16, len(os.sched_getaffinity(0)))))

    import torch

    from zero_sharded_optimizer_rank_amd import abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    abi.lib()
    if a.offload:
        return offload_main(a, w)
    if a.in_place_slot and not a.one_pass:
        print("--in-place-slot applies to the single pass only (add --one-pass)", file=sys.stderr)
        sys.exit(2)
    if a.one_pass:
        return one_pass_main(a, w)
    if w.units is not None:
        from zero_sharded_optimizer_rank_amd.units import DeviceUnits
        dev = DeviceUnits(w, a.rank)
        real = dev.real_count()
        S = dev.plan.rank_shard
        k_names = ("k1u_reduce_check", "k2u_adam")
    else:
        dev = DeviceShard(w, a.rank, **({} if a.row_align is None else {"row_align": a.row_align}))
        real = abi.zero_plan_real(dev.full_plan, a.rank)
        S = dev.count
        k_names = (("k1_reduce_check_bf16", "k2_adam_bf16") if w.dtype == "bf16"
                   else ("k1_reduce_check", "k2_adam"))
    stream = dev.stream
    n = w.world_size
    n_units = getattr(dev, "n_units", None)
    other_sq = w.other_sq(real) if w.other_ranks_from_config else 0.0
    t_setup = time.perf_counter()
    dev.load_initial_state()
    dev.load_contributions(1, w.loss_scale0)
    setup_s = time.perf_counter() - t_setup

    def args_for(t):
        return dev.args(t, w.loss_scale0, other_sq=other_sq)

    for i in range(a.warmup):
        dev.reduce_check(args_for(i + 1))
        dev.adam_apply(args_for(i + 1))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        args = args_for(a.warmup + i + 1)
        ev[i][0].record(stream)
        dev.reduce_check(args)
        ev[i][1].record(stream)
        dev.adam_apply(args)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res = dev.result()
    if res.skip:
        raise RuntimeError("a timed step was skipped")
    k1_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / a.steps
    k2_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / a.steps
    ms_per_step = wall * 1e3 / a.steps
    per_step = sorted(e[0].elapsed_time(e[2]) for e in ev)

    def pct(q):
        return per_step[min(len(per_step) - 1, int(q * len(per_step)))]

    skipped = None
    if a.time_skip:
        # skipped steps, each as zero_reduce_adam_step (or its unit / bf16 form)
        # enqueues it: (1) another rank overflowed, known on the host, so the
        # update is not launched; (2) this rank's own contributions hold an
        # inf, found on the device, so the update kernel starts and exits
        def time_skips(other):
            sk = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            args = dev.args(a.warmup + a.steps + 1, w.loss_scale0, other_sq=other_sq,
                            other_overflow=other)
            sk[0].record(stream)
            for _ in range(3):
                dev.step(args)
            sk[1].record(stream)
            torch.cuda.synchronize()
            if not dev.result().skip:
                raise RuntimeError("the forced skip was not taken")
            return sk[0].elapsed_time(sk[1]) / 3

        other_ms = time_skips(True)
        row0 = dev.contrib[0] if n_units is None else dev.bufs[0]["contrib"][0]
        keep = row0[0].item()
        row0[0] = 0x7F80 if w.dtype == "bf16" else 0x7C00  # +inf in rank 0's first element
        torch.cuda.synchronize()
        own_ms = time_skips(False)
        row0[0] = keep
        torch.cuda.synchronize()
        skipped = {"other_rank_ms": other_ms, "own_overflow_ms": own_ms,
                   "bytes_per_param": 2 * n + 4,
                   "gbps_other_rank": (2 * n + 4) * S / (other_ms * 1e6)}

    b1, b2 = bytes_per_param(n)
    kernels = {
        k_names[0]: {"ms": k1_ms, "bytes_per_param": b1, "bytes": b1 * S,
                     "gbps": b1 * S / (k1_ms * 1e6)},
        k_names[1]: {"ms": k2_ms, "bytes_per_param": b2, "bytes": b2 * S,
                     "gbps": b2 * S / (k2_ms * 1e6)},
    }
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    traffic = traffic_for(w.name, dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["gbps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": kernels[dom]["gbps"] / HBM_PEAK_GBPS, "traffic": traffic}

    del dev
    calib = calibration_copy(a.calib_bytes, stream)

    out = {
        "metric": "params updated/sec + achieved HBM GB/s, Llama-3-8B shard step N=8"
        if w.name == "llama3_8b" and not a.no_clip
        else f"params updated/sec + achieved HBM GB/s, {w.name} shard step",
        "value": real / (ms_per_step / 1e3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: rank {a.rank} of N={n}, shard S={S} "
                               f"(psi={w.psi}), {w.dtype} contributions and slot, fp32 master/m/v"
                               + (f", {n_units} FSDP units" if w.units else "")
                               + (", clipping turned off" if a.no_clip else ""),
                   "world_size_simulated": n, "shard": S, "psi": w.psi},
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "skipped_step": skipped,
        "hbm_gbps_step": (2 * n + 34) * S / (ms_per_step * 1e6),
        "hbm_gbps_step_floor_bytes": (2 * n + 26) * S / (ms_per_step * 1e6),
        "roofline": roofline,
        "kernels": kernels,
        "calibration_copy": calib,
        "setup_s": setup_s,
        "kernel_hash": kernel_hash(),
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def one_pass_main(a, w):
    """One JSON line for the single-pass step (steps without clipping)."""
    import torch
    from zero_sharded_optimizer_rank_amd import abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    if w.max_grad_norm > 0:
        print("--one-pass takes a workload without clipping (add --no-clip to turn "
              "a workload's clipping off)", file=sys.stderr)
        sys.exit(2)
    if w.units is not None:
        from zero_sharded_optimizer_rank_amd.units import DeviceUnits
        kname = "k12u_reduce_adam"
        dev = DeviceUnits(w, a.rank, one_pass=True, in_place_slot=a.in_place_slot)
        real, S = dev.real_count(), dev.plan.rank_shard
    else:
        kname = "k12_reduce_adam_bf16" if w.dtype == "bf16" else "k12_reduce_adam"
        dev = DeviceShard(w, a.rank, one_pass=True)
        real, S = abi.zero_plan_real(dev.full_plan, a.rank), dev.count
    n, stream = w.world_size, dev.stream
    other_sq = w.other_sq(real) if w.other_ranks_from_config else 0.0
    t_setup = time.perf_counter()
    dev.load_initial_state()
    dev.load_contributions(1, w.loss_scale0)
    setup_s = time.perf_counter() - t_setup
    # one result word per timed step, checked after the timed region: every
    # step must have applied, so adopting each new set unconditionally is right
    res = torch.zeros((a.warmup + a.steps, abi.RESULT_BYTES), dtype=torch.uint8,
                      device=dev.device)
    in_place = a.in_place_slot

    def one_step(t, r):
        if in_place and w.units is not None:  # the unit tables already point at the live slots
            dev.step_1pass(dev.args(t, w.loss_scale0, other_sq=other_sq), res=r)
            dev.restore_slot(res=r)
        elif in_place:
            dev.step_1pass(dev.args(t, w.loss_scale0, other_sq=other_sq), res=r,
                           in_place_slot=True)
            dev.restore_slot(res=r)
        else:
            dev.step_1pass(dev.args(t, w.loss_scale0, other_sq=other_sq), res=r)

    def adopt():
        if w.units is None:
            dev.adopt(swap_slot=not in_place)
        else:
            dev.adopt()

    for i in range(a.warmup):
        one_step(i + 1, res[i])
        adopt()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        ev[i][0].record(stream)
        one_step(a.warmup + i + 1, res[a.warmup + i])
        ev[i][1].record(stream)
        adopt()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    raw = res.cpu().numpy()
    if any(abi.zero_step_result_t.from_buffer_copy(raw[i].tobytes()).skip
           for i in range(raw.shape[0])):
        raise RuntimeError("a step was skipped")
    ms = wall * 1e3 / a.steps
    k_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / a.steps
    per_step = sorted(e[0].elapsed_time(e[1]) for e in ev)
    n_units = getattr(dev, "n_units", None)
    del dev
    calib = calibration_copy(a.calib_bytes, stream)
    bpp = 2 * n + 26
    gbps = bpp * S / (k_ms * 1e6)
    out = {
        "metric": f"params updated/sec + achieved HBM GB/s, {w.name} shard step, single pass",
        "value": real / (ms / 1e3), "unit": "params/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: rank {a.rank} of N={n}, shard S={S} (psi={w.psi}), "
                               f"{w.dtype} contributions and slot, fp32 master/m/v in two sets, "
                               f"single-pass step"
                               + (f", {n_units} FSDP units" if w.units else "")
                               + (", slot in place with zero_slot_restore each step"
                                  if in_place else "")
                               + (" (clipping turned off)" if a.no_clip else " (no clipping)"),
                   "world_size_simulated": n, "shard": S, "psi": w.psi},
        "step_ms_p10_p50_p90": [per_step[int(q * (len(per_step) - 1))] for q in (0.1, 0.5, 0.9)],
        "hbm_gbps_step": bpp * S / (ms * 1e6),
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": traffic_for(w.name + "_1pass", kname)},
        "kernels": {kname: {"ms": k_ms, "bytes_per_param": bpp, "bytes": bpp * S,
                                        "gbps": gbps,
                                        "note": "event pair spans the pass and the finalize"
                                                + (" and the slot restore" if in_place else "")}},
        "calibration_copy": calib,
        "setup_s": setup_s,
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(out), flush=True)


def offload_main(a, w):
    """One JSON line for the offload form of the step (not the default line)."""
    import torch
    from zero_sharded_optimizer_rank_amd import abi
    from zero_sharded_optimizer_rank_amd.shard import OffloadShard

    dev = OffloadShard(w, a.rank, chunk=1 << 22, threads=a.threads or None,
                       two_streams=not a.one_stream)
    real = abi.zero_plan_real(dev.full_plan, a.rank)
    S, n = dev.count, w.world_size
    other_sq = w.other_sq(real) if w.other_ranks_from_config else 0.0
    dev.load_initial_state()
    dev.load_contributions(1, w.loss_scale0)
    stream = dev.stream
    for i in range(a.warmup):
        dev.reduce_check(dev.args(i + 1, w.loss_scale0, other_sq=other_sq))
        dev.adam_apply(dev.args(i + 1, w.loss_scale0, other_sq=other_sq))
    k1_ms, host_s = [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        args = dev.args(a.warmup + i + 1, w.loss_scale0, other_sq=other_sq)
        ev[0].record(stream)
        dev.reduce_check(args)
        ev[1].record(stream)
        t1 = time.perf_counter()
        res = dev.adam_apply(args)  # waits for the reduce, then runs the pipeline
        host_s.append(time.perf_counter() - t1)
        k1_ms.append(ev[0].elapsed_time(ev[1]))
        if res.skip:
            raise RuntimeError("a timed step was skipped")
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / a.steps
    k1 = sum(k1_ms) / a.steps
    pipe = sum(host_s) / a.steps - k1 / 1e3
    b1, _ = bytes_per_param(n)
    out = {
        "metric": "params updated/sec, offload form of the shard step (host Adam, PCIe)",
        "value": real / (ms / 1e3), "unit": "params/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: rank {a.rank} of N={n}, shard S={S}, fp16 contributions "
                               f"and slot on the GPU, fp32 master/m/v in host memory, "
                               f"{dev.threads} host threads, 4M-element PCIe chunks, "
                               + ("one stream" if a.one_stream else "upload on a second stream"),
                   "world_size_simulated": n, "shard": S, "psi": w.psi},
        "roofline": {"bound": "pcie", "kernel": "offload pipeline",
                     "achieved": 6 * S / (pipe * 1e9), "peak": 64.0, "unit": "GB/s",
                     "frac": 6 * S / (pipe * 1e9) / 64.0, "traffic": None},
        "offload": {"k1_ms": k1, "pipeline_ms": pipe * 1e3,
                    "pcie_gbps": 6 * S / (pipe * 1e9),
                    "host_state_gbps": 30 * S / (pipe * 1e9),
                    "k1_gbps": b1 * S / (k1 * 1e6)},
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
