#!/usr/bin/env python3
"""Throughput of the blockwise-FP8 ZeRO-1 shard step on one MI355X.

One step = the whole per-step path on one rank's shard: fold of the reduced
row-major FP32 grads -> statistics (when clipping or loss scaling is on) ->
finalize -> AdamW + per-block amax + E4M3 requant -> unfold of the FP8 codes
and scales to row-major.  Headline route (default): the update reads the
row-major grads itself (the grad fold happens on read, no folded grad copy);
the route with a separate fold kernel is timed in the same run and reported
under `alt_mode`.  Inputs (row-major grads, folded master/m/v, state) are
resident in HBM before timing starts.

Default workload: the MoE expert shard -- params [64,2048,7168] x2 and
[64,7168,2048] FP32, block-wise split over DP = 8, rank 5 (352,321,536 real
elements), grads N(0,1e-4) x lognormal(0,1) per expert, no clipping.

Prints one JSON line (rank 0).  `value` = real elements of the shard updated
per second.  `roofline` is for the dominant call (fp8z1_step_rowmajor or
fp8z1_step: the update kernel plus its one-workgroup finalize kernel, and the
statistics pass when one runs), timed with HIP events on the stream the
kernels run on; `cpu_baseline` is the numpy oracle on a bounded sample of the
same shard.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BLOCK = 128 * 128

# Algorithmic bytes per real element (and per slot) of each call: what each kernel
# must read and write once (padding excluded), not what it happens to move.
BYTES_FOLD_F32 = 8  # read 4, write 4
BYTES_STATS = 4  # separate statistics kernel (not used when fused into the fold)
BYTES_UPDATE = 29  # read g, p, m, v (16); write p, m, v (12) + code (1)
BYTES_UNFOLD_E4M3 = 2  # read code, write code
SLOT_BYTES_UPDATE = 32 + 4  # slot plan record + scale
SLOT_BYTES_FOLD = 32 + 8  # slot plan record + the slot's float64 sum of squares
SLOT_BYTES_UNFOLD = 32 + 8  # slot plan record + scale read and write


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gen_params(w, held, make, dtype):
    import torch
    out = []
    jobs = []
    for pid, (E, R, C) in enumerate(w.shapes):
        if pid not in held:
            out.append(None)
            continue
        t = torch.zeros((E, R, C), dtype=dtype, device="cuda")
        out.append(t)
        jobs += [(pid, e) for e in held[pid]]

    def one(job):
        pid, e = job
        return job, make(pid, e)

    with ThreadPoolExecutor(_threads()) as ex:
        for (pid, e), slab in ex.map(one, jobs):
            src = torch.from_numpy(slab.view(np.int16) if dtype == torch.bfloat16 else slab)
            if dtype == torch.bfloat16:
                src = src.view(torch.bfloat16)
            out[pid][e].copy_(src)
    return out


def _held(entries):
    held = {}
    for p, e in zip(entries["param"], entries["expert"]):
        if p >= 0:
            held.setdefault(int(p), set()).add(int(e))
    return {p: sorted(s) for p, s in held.items()}


def _update_kernel_names(entries, mode: str) -> str:
    """The update kernels fp8z1_step* launches on this shard: the 1024-lane full-block
    kernel over the full blocks when there are at least 8,192 of them, the general
    kernel over the rest (partial blocks, padding slots, or a small shard)."""
    g = "<rowmajor>" if mode == "fold_on_read" else "<folded>"
    full = int(((entries["vrows"] == 128) & (entries["vcols"] == 128) & (entries["param"] >= 0)).sum())
    other = len(entries) - full
    names = []
    if full >= 8192:
        names.append("update_full_kernel" + g)
    if other or full < 8192:
        names.append("update_kernel" + g)
    return " + ".join(names)


def _source_hash() -> str:
    """Hash of the kernel sources with comments and blank space taken out, so
    that it changes when the code does and not when only its comments do."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "blockwise_fp8_zero_fold_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            text = open(os.path.join(csrc, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str, mode: str, src_hash: str, split: str = ""):
    """HBM bytes (read + written) per launch of the dominant kernel from the committed
    rocprofv3 counter summary of this workload (and split, when it is not the
    workload's own), or None when there is none or the kernels changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"update_kernel_{workload}{split}_{mode}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, rank: int, slots: int, steps: int = 2, first: int = 0):
    """The oracle (numpy, as committed) on a bounded sample of the same shard: per step
    fold of the grads, the step, unfold of the codes, over ``slots`` slots from ``first``."""
    from oracle import layout, optim, step, table

    tab = table.build(w.shapes, w.dp, rank, table.PARAM if w.split == "param" else table.BLOCK)
    sub = dict(tab)
    sub["entries"] = tab["entries"][first:first + slots]
    slots = len(sub["entries"])
    sub["shard_slots"] = slots
    held = _held(sub["entries"])
    G = {p: np.zeros(w.shapes[p], np.float32) for p in held}
    P = {p: np.zeros(w.shapes[p], np.float32) for p in held}
    for p, es in held.items():
        for e in es:
            G[p][e] = synth.grad_slab(w, p, e, 1)
            P[p][e] = synth.master_slab(w, p, e)
    master = layout.fold_shard(sub, P)
    n = slots
    z = np.zeros((n, 128, 128), np.float32)
    codes = np.zeros((n, 128, 128), np.uint8)
    sc = np.zeros(n, np.float32)
    out = {p: np.zeros(w.shapes[p], np.uint8) for p in held}
    m, v, st = z, z.copy(), optim.init_state(w.hp)
    t0 = time.perf_counter()
    for _ in range(steps):
        g = layout.fold_shard(sub, G)
        st, master, m, v, codes, sc = step.step_sharded(sub, w.hp, st, g, master, m, v, codes, sc)
        layout.unfold_shard(sub, codes, out)
    dt = (time.perf_counter() - t0) / steps
    valid = int(np.sum(sub["entries"]["vrows"].astype(np.int64) * sub["entries"]["vcols"]))
    return valid / dt, valid, dt


def _cpu_worker(job):
    """One worker of the parallel oracle run (a fresh process, no GPU use)."""
    name, split, rank, first, slots, steps, barrier = job
    w = synth.get(name).with_(split=split)
    barrier.wait()
    t0 = time.perf_counter()
    rate, valid, dt = cpu_baseline(w, rank, slots, steps=steps, first=first)
    return valid, dt, time.perf_counter() - t0


def cpu_baseline_parallel(w, rank: int, nslots: int, procs: int, steps: int = 2):
    """The same oracle in ``procs`` worker processes, each on its own contiguous slot
    range, together covering the whole shard; elements/s = real elements of the shard
    / the slowest worker's time per step.  Workers start from a clean interpreter
    (spawn) and never touch the GPU; each keeps its own clipping statistics (the
    timed work is the same)."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    per = -(-nslots // procs)
    ranges = [(i * per, min(per, nslots - i * per)) for i in range(procs) if i * per < nslots]
    mgr = ctx.Manager()
    barrier = mgr.Barrier(len(ranges))
    with ctx.Pool(len(ranges)) as pool:
        res = pool.map(_cpu_worker, [(w.name, w.split, rank, a, n, steps, barrier) for a, n in ranges])
    mgr.shutdown()
    valid = sum(r[0] for r in res)
    dt = max(r[1] for r in res)
    return valid / dt, valid, dt, len(ranges)


def _host_info() -> dict:
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_visible": os.cpu_count()}


def _table_info(w, rank: int) -> dict:
    """Host table build time and padding of both splits (the reason for the param split
    is less padding per rank; its cost is every rank padded to the largest bucket)."""
    import blockwise_fp8_zero_fold_amd as fz
    out = {}
    for name, split in (("block", fz.SPLIT_BLOCK), ("param", fz.SPLIT_PARAM)):
        t0 = time.perf_counter()
        t = fz.fp8z1_build_table(w.shapes, w.dp, rank, split)
        ms = (time.perf_counter() - t0) * 1e3
        a = fz.fp8z1_build_table(w.shapes, w.dp, fz.ALL_RANKS, split)
        out[name] = {"build_ms": ms, "rank_slots": t.shard_slots,
                     "rank_pad_frac": t.info["pad_elems"] / max(1, t.shard_slots * BLOCK),
                     "all_ranks_pad_frac": a.info["pad_elems"] / max(1, a.shard_slots * BLOCK)}
        t.free()
        a.free()
    return out


def _device_info() -> dict:
    """What identifies the GPU and its memory set-up (bandwidth differs between parts):
    torch's device properties, and from the GPU's own sysfs node (matched by PCI
    address) the current clock levels, partition modes, VBIOS, VRAM vendor and power cap."""
    import glob

    import torch
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "cus": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / 2**30, 1), "l2_bytes": getattr(pr, "L2_cache_size", None)}
    uuid = getattr(pr, "uuid", None)
    if uuid is not None:
        info["uuid"] = str(uuid)
    pci = None
    if all(hasattr(pr, a) for a in ("pci_domain_id", "pci_bus_id", "pci_device_id")):
        pci = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        info["pci"] = pci
    cards = sorted(glob.glob("/sys/class/drm/card*/device"))
    dev = None
    for c in cards:
        try:
            if pci and os.path.realpath(c).endswith(pci):
                dev = c
                break
        except OSError:
            pass
    if dev is None and cards:
        dev = cards[0]
        info["sysfs_node"] = "first card (no PCI match)"

    def read(name):
        try:
            return open(os.path.join(dev, name)).read().strip()
        except (OSError, TypeError):
            return None

    if dev is not None:
        for key in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk", "pp_dpm_socclk"):  # current level marked '*'
            text = read(key)
            if text:
                cur = [ln.split(":", 1)[1].strip(" *") for ln in text.splitlines() if ln.rstrip().endswith("*")]
                if cur:
                    info[key.replace("pp_dpm_", "clock_")] = cur[0]
        for key in ("current_memory_partition", "current_compute_partition", "vbios_version",
                    "mem_info_vram_vendor"):
            v = read(key)
            if v:
                info[key] = v
        for f in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_cap"))):
            try:
                info["power_cap_w"] = int(open(f).read().strip()) / 1e6
                break
            except (OSError, ValueError):
                pass
        # temperatures (edge / junction / memory) and power right after the timed work
        for f in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "temp*_input"))):
            try:
                label = open(f.replace("_input", "_label")).read().strip()
                info[f"temp_{label}_c"] = int(open(f).read().strip()) / 1000
            except (OSError, ValueError):
                pass
        for name in ("power1_average", "power1_input"):
            for f in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", name))):
                try:
                    info["power_w"] = int(open(f).read().strip()) / 1e6
                except (OSError, ValueError):
                    pass
    return info


def sweep_ranks(w, args) -> int:
    """The fold-on-read step (update + requant, then unfold) on every rank's shard in
    turn, each with its own inputs; one JSON line with per-rank times."""
    import torch

    import blockwise_fp8_zero_fold_amd as fz
    from blockwise_fp8_zero_fold_amd.shard import Shard
    split = fz.SPLIT_PARAM if w.split == "param" else fz.SPLIT_BLOCK
    hp = fz.Hparams.make(w.hp)
    stream = torch.cuda.current_stream()
    rows = []
    for r in range(w.dp):
        sh = Shard(w.shapes, w.dp, r, split)
        held = _held(sh.table.entries())
        weights = _gen_params(w, held, lambda p, e: synth.master_slab(w, p, e), torch.float32)
        sh.init(hp, weights, fz.F32)
        del weights
        grads = _gen_params(w, held, lambda p, e: synth.grad_slab(w, p, e, 1), torch.float32)
        codes = [torch.zeros(s, dtype=torch.uint8, device="cuda") if p in held else None
                 for p, s in enumerate(w.shapes)]
        scales = [torch.zeros((s[0], -(-s[1] // 128), -(-s[2] // 128)), dtype=torch.float32, device="cuda")
                  if p in held else None for p, s in enumerate(w.shapes)]
        for _ in range(args.warmup):
            sh.step(hp, grads, codes, scales, fold_on_read=True)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e in ev:
            e[0].record(stream)
            sh.update_rowmajor(hp, grads)
            e[1].record(stream)
            sh.unfold(codes, scales)
            e[2].record(stream)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        valid = sh.table.info["valid_elems"]
        rows.append({"rank": r, "slots": sh.n_slots, "valid_elems": valid, "ms_per_step": ms,
                     "step_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
                     "unfold_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])),
                     "elems_per_s": valid / (ms * 1e-3)})
        print(f"# rank {r}: {ms:.4f} ms per step", file=sys.stderr, flush=True)
        del sh, grads, codes, scales
        torch.cuda.empty_cache()
    ms_all = sorted(x["ms_per_step"] for x in rows)
    print(json.dumps({"sweep": "ranks", "workload": w.name, "dp": w.dp, "steps": args.steps, "warmup": args.warmup,
                      "route": "fold on read", "per_rank": rows, "min_ms": ms_all[0],
                      "median_ms": float(np.median(ms_all)), "max_ms": ms_all[-1], "device": _device_info(),
                      "source_hash": _source_hash()}), flush=True)
    return 0


def next_rows(w, args) -> int:
    """The steps after the shard step, and the scale variant, on the same workload:
    the unfold of the whole all-gathered FP8 buffer (every rank's codes and scales),
    dequantization of the row-major codes to BF16 and FP32, and the shard step with
    power-of-two (E8M0) block scales beside the default rule.  One JSON line."""
    import torch

    import blockwise_fp8_zero_fold_amd as fz
    from blockwise_fp8_zero_fold_amd.shard import Shard
    split = fz.SPLIT_PARAM if w.split == "param" else fz.SPLIT_BLOCK
    stream = torch.cuda.current_stream()

    def ev_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    # whole gathered buffer: codes and scales of all ranks in rank order
    tall = fz.fp8z1_build_table(w.shapes, w.dp, fz.ALL_RANKS, split)
    n_all, valid_all = tall.shard_slots, tall.info["valid_elems"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    folded = torch.randint(0, 256, (n_all * BLOCK,), dtype=torch.uint8, device="cuda", generator=gen)
    fsc = torch.rand(n_all, dtype=torch.float32, device="cuda", generator=gen)
    codes = [torch.empty(s, dtype=torch.uint8, device="cuda") for s in w.shapes]
    scales = [torch.empty((s[0], -(-s[1] // 128), -(-s[2] // 128)), dtype=torch.float32, device="cuda")
              for s in w.shapes]
    ms = ev_ms(lambda: fz.fp8z1_unfold(tall, folded, fz.E4M3, fsc, codes, scales), args.steps)
    nbytes = 2 * valid_all + SLOT_BYTES_UNFOLD * n_all
    out["whole_buffer_unfold"] = {"slots": n_all, "valid_elems": valid_all, "ms": ms,
                                  "gbs_algorithmic": nbytes / (ms * 1e-3) / 1e9,
                                  "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    print(f"# whole-buffer unfold: {ms:.4f} ms", file=sys.stderr, flush=True)
    del folded, fsc
    # dequantization of every param's row-major codes
    for name, dt, tdt, el in (("dequantize_bf16", fz.BF16, torch.bfloat16, 2), ("dequantize_f32", fz.F32,
                                                                                 torch.float32, 4)):
        big = max(int(np.prod(s)) for s in w.shapes)
        buf = torch.empty(big, dtype=tdt, device="cuda")

        def deq():
            for p, s in enumerate(w.shapes):
                fz.fp8z1_dequantize(codes[p], scales[p], s, dt, buf[:int(np.prod(s))].view(s))
        ms = ev_ms(deq, args.steps)
        tot = sum(int(np.prod(s)) for s in w.shapes)
        nbytes = (1 + el) * tot
        out[name] = {"elems": tot, "ms": ms, "gbs_algorithmic": nbytes / (ms * 1e-3) / 1e9,
                     "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        print(f"# {name}: {ms:.4f} ms", file=sys.stderr, flush=True)
        del buf
    tall.free()
    del codes, scales
    torch.cuda.empty_cache()
    # the shard step with each scale rule
    rank = w.ranks[0]
    sh = Shard(w.shapes, w.dp, rank, split)
    held = _held(sh.table.entries())
    weights = _gen_params(w, held, lambda p, e: synth.master_slab(w, p, e), torch.float32)
    grads = _gen_params(w, held, lambda p, e: synth.grad_slab(w, p, e, 1), torch.float32)
    rc = [torch.zeros(s, dtype=torch.uint8, device="cuda") if p in held else None for p, s in enumerate(w.shapes)]
    rs = [torch.zeros((s[0], -(-s[1] // 128), -(-s[2] // 128)), dtype=torch.float32, device="cuda")
          if p in held else None for p, s in enumerate(w.shapes)]
    valid = sh.table.info["valid_elems"]
    for rule_name, rule in (("amax", 0), ("pow2", 1)):
        hp = fz.Hparams.make(dataclasses.replace(w.hp, scale_rule=rule))
        sh.init(hp, weights, fz.F32)
        ms = ev_ms(lambda: sh.step(hp, grads, rc, rs, fold_on_read=True), args.steps)
        out[f"step_scale_{rule_name}"] = {"ms": ms, "elems_per_s": valid / (ms * 1e-3)}
        print(f"# step with {rule_name} scales: {ms:.4f} ms", file=sys.stderr, flush=True)
    print(json.dumps({"next_rows": out, "workload": w.name, "dp": w.dp, "rank": rank, "steps": args.steps,
                      "device": _device_info(), "source_hash": _source_hash()}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="moe", choices=["moe", "dense", "full", "ragged"])
    ap.add_argument("--split", default=None, choices=["block", "param"], help="override the workload's split")
    ap.add_argument("--mode", default="fold_on_read", choices=["fold_on_read", "fold"],
                    help="headline route: the update reads the row-major grads (fold on read), or a separate "
                         "fold kernel writes folded grads first; the other route is timed too and reported "
                         "under alt_mode")
    ap.add_argument("--unfused-stats", action="store_true", help="separate statistics kernel instead of fold-fused")
    ap.add_argument("--cpu-slots", type=int, default=16384, help="oracle sample size (slots) for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--next-rows", action="store_true",
                    help="time the whole-buffer unfold, dequantization and the E8M0-scale step on the workload and "
                         "print one JSON line; not the headline line")
    ap.add_argument("--sweep-ranks", action="store_true",
                    help="time the fold-on-read step on every rank's shard of the workload in turn and print one "
                         "JSON line with per-rank times (min / median / max); not the headline line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run torch's plain copy of 2 x 1 GiB five times (the reference kernel whose "
                         "FETCH_SIZE/WRITE_SIZE counters calibrate the HBM traffic of the step kernels)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}): the path runs one data-parallel rank's "
              "shard; collectives across GPUs are not part of it", file=sys.stderr)
        return 2

    w = synth.get(args.workload)
    if args.split:
        w = w.with_(split=args.split)
    rank = w.ranks[0]

    # The oracle baselines run first, before this process touches the GPU (the
    # parallel one starts worker processes).
    cpu = cpu_par = None
    if not (args.no_cpu_baseline or args.calibrate_copy or args.sweep_ranks or args.next_rows):
        from oracle import table as otable
        n_all = otable.build(w.shapes, w.dp, rank, otable.PARAM if w.split == "param" else otable.BLOCK)["shard_slots"]
        slots = min(args.cpu_slots, n_all)
        print(f"# cpu baseline: oracle on {slots} slots, one process", file=sys.stderr, flush=True)
        rate, n_el, dt = cpu_baseline(w, rank, slots, steps=2)
        cpu = {"value": rate, "unit": "elements/s", "cores": 1, "kind": "oracle",
               "sample": f"2 steps of fold+step+unfold over the first {slots} slots ({n_el} real elements) of the "
                         f"same shard, numpy, one thread, {dt:.1f}s per step", "host": _host_info()}
        procs = _threads()
        print(f"# cpu baseline: oracle on all {n_all} slots, {procs} processes", file=sys.stderr, flush=True)
        rate, n_el, dt, used = cpu_baseline_parallel(w, rank, n_all, procs, steps=2)
        cpu_par = {"value": rate, "unit": "elements/s", "cores": used, "kind": "oracle",
                   "sample": f"2 steps of fold+step+unfold over the whole shard ({n_el} real elements), split into "
                             f"{used} contiguous slot ranges, one numpy process each, {dt:.2f}s per step (slowest "
                             "process)", "host": _host_info()}

    import torch

    if args.calibrate_copy:
        n = 1 << 28  # 1 GiB of float32
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy": {"bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                                             "launches": 5}}), flush=True)
        return 0

    import blockwise_fp8_zero_fold_amd as fz
    from blockwise_fp8_zero_fold_amd.shard import Shard

    if args.sweep_ranks:
        return sweep_ranks(w, args)
    if args.next_rows:
        return next_rows(w, args)
    split = fz.SPLIT_PARAM if w.split == "param" else fz.SPLIT_BLOCK
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    sh = Shard(w.shapes, w.dp, rank, split)
    info = sh.table.info
    valid = info["valid_elems"]
    nslots = info["shard_slots"]
    held = _held(sh.table.entries())
    print(f"# setup: {w.name} rank {rank}: {nslots} slots, {valid} real elements", file=sys.stderr, flush=True)
    if w.master_dtype == "bf16":
        weights = _gen_params(w, held, lambda p, e: synth.master_slab_bf16(w, p, e), torch.bfloat16)
        wdt = fz.BF16
    else:
        weights = _gen_params(w, held, lambda p, e: synth.master_slab(w, p, e), torch.float32)
        wdt = fz.F32
    sh.init(fz.Hparams.make(w.hp), weights, wdt)
    # the init fold of the weights into the FP32 master (once per run; timed
    # here on the same weights, which leaves the master as it was)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(torch.cuda.current_stream())
    for _ in range(3):
        fz.fp8z1_fold(sh.table, weights, wdt, sh.master)
    ev1.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    init_fold_ms = ev0.elapsed_time(ev1) / 3
    init_fold = {"dtype": "bf16" if wdt == fz.BF16 else "f32", "ms": init_fold_ms,
                 "gbs_algorithmic": ((2 if wdt == fz.BF16 else 4) + 4) * info["valid_elems"] / (init_fold_ms * 1e-3) / 1e9}
    del weights
    grads = _gen_params(w, held, lambda p, e: synth.grad_slab(w, p, e, 1), torch.float32)
    codes = [torch.zeros(s, dtype=torch.uint8, device="cuda") if p in held else None for p, s in enumerate(w.shapes)]
    scales = [torch.zeros((s[0], -(-s[1] // 128), -(-s[2] // 128)), dtype=torch.float32, device="cuda")
              if p in held else None for p, s in enumerate(w.shapes)]
    hp = fz.Hparams.make(w.hp)
    stats = w.hp.max_grad_norm > 0 or w.hp.loss_scaling
    fused = stats and not args.unfused_stats
    torch.cuda.synchronize()
    print(f"# setup done in {time.perf_counter() - t_setup:.1f}s; warmup {args.warmup}, timed {args.steps}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def one_step(mode, ev=None, i=0):
        def rec(name, which):
            if ev is not None:
                ev[name][which][i].record(stream)
        if mode == "fold_on_read":
            rec("step", 0)
            sh.update_rowmajor(hp, grads)
            rec("step", 1)
        else:
            rec("fold", 0)
            pre = sh.fold_grads(hp, grads, fused_stats=fused)
            rec("fold", 1)
            rec("step", 0)
            sh.update(hp, presummed=pre)
            rec("step", 1)
        rec("unfold", 0)
        sh.unfold(codes, scales)
        rec("unfold", 1)

    medians = {}

    def timed(mode):
        for _ in range(args.warmup):
            one_step(mode)
        torch.cuda.synchronize()
        calls = ("step", "unfold") if mode == "fold_on_read" else ("fold", "step", "unfold")
        ev = {k: ([torch.cuda.Event(enable_timing=True) for _ in range(args.steps)],
                  [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]) for k in calls}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            one_step(mode, ev, i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        times = {k: [a.elapsed_time(b) for a, b in zip(*ev[k])] for k in ev}
        ms = {k: float(np.mean(v)) for k, v in times.items()}
        medians[mode] = {k: float(np.median(v)) for k, v in times.items()}
        print(f"# {mode}: {args.steps} steps in {elapsed:.3f}s; per call ms: {ms}", file=sys.stderr, flush=True)
        return elapsed * 1e3 / args.steps, ms

    def step_bytes(mode):
        """Algorithmic bytes of one whole step, and of its fp8z1_step* call."""
        call = BYTES_UPDATE * valid + SLOT_BYTES_UPDATE * nslots
        if stats and (mode == "fold_on_read" or not fused):
            call += BYTES_STATS * valid + SLOT_BYTES_FOLD * nslots
        total = call + BYTES_UNFOLD_E4M3 * valid + SLOT_BYTES_UNFOLD * nslots
        if mode == "fold":
            total += BYTES_FOLD_F32 * valid + SLOT_BYTES_FOLD * nslots
        return total, call

    def graph_timed(mode):
        """The same step captured once into a HIP graph, replayed K times."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_step(mode)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        print(f"# {mode} as a graph: {args.steps} replays in {elapsed:.3f}s", file=sys.stderr, flush=True)
        return elapsed * 1e3 / args.steps

    modes = [args.mode, "fold" if args.mode == "fold_on_read" else "fold_on_read"]
    results = {m: timed(m) for m in modes}
    headline_medians = dict(medians[args.mode])  # before the skipped-step timing reuses the route
    graph_ms = graph_timed(args.mode)

    skip = None
    if stats:
        # a skipped step (overflow reported by the other ranks): statistics and
        # finalize run, the update exits at once, the unfold rewrites the codes
        hp_run = hp
        hp = fz.Hparams.make(w.hp, extra_found_inf=True)
        _, skip_calls = timed(args.mode)
        hp = hp_run
        skip = {"mode": args.mode, "per_call_ms": skip_calls,
                "note": "skipped steps (overflow flag from the other ranks): statistics + finalize, no update"}
    st = sh.read_state()
    print(f"# state step {st['step']}", file=sys.stderr, flush=True)

    ms_per_step, ms = results[args.mode]
    total_bytes, call_bytes = step_bytes(args.mode)
    achieved = call_bytes / (ms["step"] * 1e-3) / 1e9
    src_hash = _source_hash()
    traffic_split = "" if w.split == synth.get(w.name).split else f"_{w.split}"
    alt_mode = modes[1]
    alt_ms, alt_calls = results[alt_mode]
    alt_total, _ = step_bytes(alt_mode)

    # streaming references measured in the same run: the update's access pattern
    # with no arithmetic (same slots, same bytes), and a plain 4 KB-per-workgroup copy
    def ev_time(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    probe_bufs = [torch.zeros(nslots * BLOCK, dtype=torch.float32, device="cuda") for _ in range(4)]
    probe_codes = torch.zeros(nslots * BLOCK, dtype=torch.uint8, device="cuda")
    pat_bytes = 29 * nslots * BLOCK
    pat_gbs = {}
    for parts in (1, 2, 4, 8):  # 64, 32, 16, 8 KB of each array per workgroup
        t = ev_time(lambda: fz.fp8z1_probe_update_pattern(*probe_bufs, probe_codes, nslots, parts), 10)
        pat_gbs[f"{64 // parts}KB"] = pat_bytes / t / 1e9
    t_pat = pat_bytes / (pat_gbs["64KB"] * 1e9)
    t_copy = ev_time(lambda: fz.fp8z1_probe_copy(probe_bufs[0], probe_bufs[1]), 10)
    copy_bytes = 2 * probe_bufs[0].numel() * 4
    # the same copy with the workgroups in flight spread over S far-apart ranges
    tiles = probe_bufs[0].numel() * 4 // 4096
    spread_gbs = {}
    for S in (1, 16, 64, 256, 1024):
        if tiles % S == 0:
            spread_gbs[S] = copy_bytes / ev_time(lambda: fz.fp8z1_probe_copy(probe_bufs[0], probe_bufs[1], S), 10) / 1e9
    del probe_bufs, probe_codes
    torch.cuda.empty_cache()
    ceiling = {"update_pattern_gbs": pat_bytes / t_pat / 1e9, "update_pattern_gbs_by_tile": pat_gbs,
               "update_pattern_best_gbs": max(pat_gbs.values()), "copy_gbs": copy_bytes / t_copy / 1e9,
               "update_vs_pattern": achieved / (pat_bytes / t_pat / 1e9),
               "update_vs_best_pattern": achieved / max(pat_gbs.values()),
               # the second denominator beside the 8 TB/s peak: a plain device copy in the same run
               "update_vs_copy": achieved / (copy_bytes / t_copy / 1e9),
               "copy_gbs_by_spread": spread_gbs,
               "note": "same-run streaming references: fp8z1_probe_update_pattern (the update's loads and stores, "
                       "no arithmetic, same slot count) and fp8z1_probe_copy (plain copy, 4 KB per workgroup)"}
    print(f"# ceilings: update pattern {ceiling['update_pattern_gbs']:.0f} GB/s, copy {ceiling['copy_gbs']:.0f} GB/s, "
          f"copy by spread {({k: round(v) for k, v in spread_gbs.items()})}", file=sys.stderr, flush=True)

    out = {
        "metric": "optimizer-step elements/s and GB/s (% of HBM peak) per 1-GPU shard",
        "value": valid / (ms_per_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": {"moe": "moe_expert_shard", "dense": "dense_layer_set", "full": "full_step_bf16",
                         "ragged": "ragged_600_params"}[w.name],
            "shapes": [list(s) for s in w.shapes] if len(w.shapes) <= 8 else f"{len(w.shapes)} params",
            "dp": w.dp, "rank": rank, "split": w.split, "shard_slots": nslots, "valid_elems": valid,
            "clip": w.hp.max_grad_norm, "loss_scaling": bool(w.hp.loss_scaling),
            "grad_fold": "on read, inside the update" if args.mode == "fold_on_read" else "separate fold kernel",
            "stats": ("off" if not stats else
                      "separate pass over row-major grads" if args.mode == "fold_on_read" else
                      "fused into the fold" if fused else "separate pass over folded grads"),
        },
        "step_bytes": total_bytes,
        "gbs_algorithmic": total_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_step": total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "per_call_ms": ms,
        "per_call_ms_median": headline_medians,
        "roofline": {
            "kernel": _update_kernel_names(sh.table.entries(), args.mode)
                      + " + finalize_kernel" + (" + statistics pass" if stats and (args.mode == "fold_on_read" or not fused) else ""),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": _traffic(w.name, args.mode, src_hash, traffic_split),
            # where `traffic` comes from: the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of
            # this workload and route, used only while the kernel sources hash to its recorded value
            "traffic_source": (f"profiles/update_kernel_{w.name}{traffic_split}_{args.mode}_pmc.json"
                               f" (kernel sources {src_hash})"),
            "bytes_per_launch": call_bytes,
        },
        "ceiling": ceiling,
        "alt_mode": {"mode": alt_mode, "ms_per_step": alt_ms, "value": valid / (alt_ms * 1e-3),
                     "per_call_ms": alt_calls, "gbs_algorithmic": alt_total / (alt_ms * 1e-3) / 1e9},
        "skip_step": skip,
        "init_fold": init_fold,
        "graph": {"mode": args.mode, "ms_per_step": graph_ms, "value": valid / (graph_ms * 1e-3),
                  "note": "the same step captured into one HIP graph and replayed"},
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
        "table": _table_info(w, rank),
        "device": _device_info(),
        "source_hash": src_hash,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
