#!/usr/bin/env python3
"""Benchmark: one data-parallel rank's fused ZeRO-1 optimizer step on one MI355X.

A step is the whole hot path for one rank's shard: reduce the W replicas' bf16
gradient slices (fp32, rank order, / W), this rank's fp64 sum of squares, the
global-norm clip, AdamW (update, then decay) on the fp32 master/m/v, and the
bf16 parameter write-back over the ragged per-tensor list (multi-tensor apply).

Default workload: the GPT-2 small tensor list (148 tensors, 124,439,808
parameters) cut into W=8 ZeRO-1 shards; rank 4's 15,554,976-parameter shard
(31 pieces).  All inputs are synthetic (seeded) and resident in HBM before the
timed region.  The other ranks' partial sums of squares are computed once
before timing (they are what a multi-GPU run would exchange mid-step).

Memory: by default every array of the step sits in one allocation laid out by
zero1_arena_plan (the update's five streams 40 GiB apart; HBM serves them
faster than arrays packed together); --layout packed allocates each array on
its own.

Prints ONE JSON line.  Metric: shard parameters updated per second; the
algorithmic HBM traffic is (2W+26) bytes per parameter (W bf16 gradient reads,
fp32 master/m/v read + write, bf16 parameter write).

Modes:
  python bench.py [--steps K] [--warmup W] [--config C2]    the benchmark line
  python bench.py --pmc-run                                   short run for rocprofv3 --pmc
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR OUT     counter summary for profiles/
                 [--pmc-also KERNEL]                          (and of another kernel of the step)
  python bench.py --summarize-kt KT_DIR OUT                   kernel-trace summary for profiles/
"""
from __future__ import annotations

import argparse
import glob
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
UPDATE_KERNEL = "adamw_mta_kernel"
ONCHIP_KERNEL = "onchip_step_kernel"
REDUCE_KERNEL = "reduce_kernel"
CALIB_BYTES = 1 << 30          # the plain copy used to scale the PMC byte counters
PMC_SUMMARY = os.path.join(ROOT, "profiles", "adamw_mta_kernel_gpt2small_w8_pmc.txt")


def kernel_source_hash() -> str:
    """Hash of the library's sources with comments and blank space removed: it
    changes when the code changes, not when a comment does."""
    import re
    h = hashlib.sha256()
    for p in ("zero_sharded_mixed_zero1_amd/csrc/kernels.hip", "zero_sharded_mixed_zero1_amd/csrc/internal.h",
              "zero_sharded_mixed_zero1_amd/csrc/api.cpp"):
        with open(os.path.join(ROOT, p)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------- setup
class Copy:
    """One independent copy of everything a step touches (rotated through so
    that consecutive steps do not find each other's data in the 256 MB MALL)."""


def setup(torch, cfg, design_flags, n_copies, dev, layout="arena", arena_all=False, arena_offset=0):
    """Every array of n_copies independent copies of one rank's step, resident
    in HBM.  layout "arena": one allocation laid out by zero1_arena_plan (the
    update's five streams 40 GiB apart, the gradient buffers packed after
    them); copy c sits c * delta bytes after copy 0, inside copy 0's gaps.
    layout "packed": one torch allocation per array."""
    import synth
    import zero_sharded_mixed_zero1_amd as z

    W, rank = cfg.W, cfg.rank
    numels = [n for _, n in cfg.tensors]
    N = sum(numels)
    begin, S = z.shard_range(N, W, rank)
    pieces_l = z.shard_pieces(numels, begin, begin + S)
    offsets = [0]
    for n in numels:
        offsets.append(offsets[-1] + n)
    first, last = pieces_l[0][0], pieces_l[-1][0]
    p_lo, p_hi = offsets[first], offsets[last + 1]      # the tensors the shard touches
    grad_elems, grad_off = (N, begin) if cfg.all_replicas_resident else (S, 0)
    mvdt = torch.int16 if cfg.mv_bf16 else torch.float32
    mv_flag = z.MV_BF16 if cfg.mv_bf16 else 0
    arena = None
    info = {"layout": layout}
    if layout == "arena":
        free, _ = torch.cuda.mem_get_info(dev)
        cap = max(0, free - (8 << 30))
        try:
            L = z.arena_plan(S, W, grad_elems, grad_off, p_hi - p_lo, begin - p_lo,
                             flags=mv_flag | (design_flags & (z.STORE_G | z.RECOMPUTE_G)), capacity=cap)
        except z.Zero1Error as e:
            L = None
            info.update(layout="packed", arena_refused=e.message)
        if L is not None:
            unit = 2 << 20
            # copy c is copy 0 shifted by c * delta: delta clears the largest spaced
            # array and the whole region from the parameter buffer to the end
            extents = [L.ws_bytes, 4 * S, (2 if cfg.mv_bf16 else 4) * S]
            delta = (max(extents + [L.total_bytes - L.params]) + unit - 1) // unit * unit
            total = L.total_bytes + (n_copies - 1) * delta
            if n_copies > 1 and delta * (n_copies - 1) + max(extents) + 2 * (begin - p_lo) > L.spacing:
                L = None
                info.update(layout="packed", arena_refused="the rotated copies do not fit in the arena's gaps")
        layout = info["layout"]
    if layout == "arena":
        base = (int(arena_offset) >> 21) << 21
        if arena_all:   # the arena takes all free memory (less 8 GB), as a preallocating allocator would
            if base + total > cap:
                raise SystemExit("arena: the offset layout does not fit in the free memory")
            total = max(base + total, cap)
        arena = torch.empty(total, dtype=torch.uint8, device=dev)[base:]
        info.update(arena_bytes=total, spacing_gib=L.spacing / (1 << 30))
        spans = []

        def view(off, n, dt):
            nb = n * torch.empty((), dtype=dt).element_size()
            spans.append((off, off + nb))
            return arena[off:off + nb].view(dt)
    copies = []
    for c in range(n_copies):
        cp = Copy()
        if layout == "arena":
            sh = c * delta
            bufs = [view(sh + L.grads[w], grad_elems, torch.int16) for w in range(W)]
            cp.master = view(sh + L.master, S, torch.float32)
            cp.m = view(sh + L.m, S, mvdt)
            cp.v = view(sh + L.v, S, mvdt)
            cp.params = view(sh + L.params, p_hi - p_lo, torch.int16)
            cp.ws = view(sh + L.ws, L.ws_bytes, torch.uint8)
        else:
            bufs = [torch.empty(grad_elems, dtype=torch.int16, device=dev) for _ in range(W)]
            cp.master = torch.empty(S, dtype=torch.float32, device=dev)
            cp.m = torch.empty(S, dtype=mvdt, device=dev)
            cp.v = torch.empty(S, dtype=mvdt, device=dev)
            cp.params = torch.empty(p_hi - p_lo, dtype=torch.int16, device=dev)
            cp.ws = None
        for w, t in enumerate(bufs):
            synth.fill_bf16_(t, synth.grad_key(cfg.seed, 1, w), begin - grad_off, cfg.sigma, cfg.outlier_pct)
        if cfg.all_replicas_resident:
            # every replica's full flat gradient is resident; the step reads rank's slice
            cp.full = bufs
            cp.begin = begin
        else:
            # only this rank's W slices exist (their global flat indices start at begin)
            cp.begin = 0
        cp.grads = bufs
        synth.fill_f32_(cp.master, synth.master_key(cfg.seed), begin, cfg.master_sigma)
        cp.m.zero_()
        cp.v.zero_()
        cp.params.zero_()
        # the model's bf16 parameters of the tensors the shard touches (pieces point inside)
        pieces = [(n, so, cp.params[offsets[ti] - p_lo + off:], cp.master[so:], cp.m[so:], cp.v[so:])
                  for ti, off, so, n in pieces_l]
        cp.table = torch.empty(max(256, z.mta_table_bytes(pieces)), dtype=torch.uint8, device=dev)
        cp.plan = z.mta_plan(pieces, cp.table, flags=mv_flag)
        if cp.ws is None or cp.ws.numel() < z.mta_workspace_bytes(cp.plan, W, design_flags):
            cp.ws = torch.empty(z.mta_workspace_bytes(cp.plan, W, design_flags), dtype=torch.uint8, device=dev)
        cp.rsd = torch.zeros(W, dtype=torch.float64, device=dev)
        copies.append(cp)
    if arena is not None:   # no two arrays of any copy overlap (checked before any step runs)
        spans.sort()
        for (a0, b0), (a1, b1) in zip(spans, spans[1:]):
            if b0 > a1:
                raise SystemExit(f"arena: arrays overlap at byte {a1}")
    # the other ranks' partial sums of squares (C1/C2: all replicas resident -> true global norm;
    # otherwise only this rank's slices exist and the other partials are 0: shard-local norm)
    if cfg.all_replicas_resident:
        c0 = copies[0]
        wsr = torch.empty(z.workspace_bytes(S + 8, W), dtype=torch.uint8, device=dev)
        for r in range(W):
            b, n = z.shard_range(N, W, r)
            z.shard_reduce(c0.full, b, n, sumsq_out=c0.rsd[r:r + 1], ws=wsr)
        torch.cuda.synchronize()
        for cp in copies[1:]:
            cp.rsd.copy_(c0.rsd)
    torch.cuda.synchronize()
    return dict(W=W, rank=rank, N=N, S=S, begin=begin, pieces=len(pieces_l), copies=copies, info=info)


def hp(cfg, t):
    return cfg.hparams(t)


# ---------------------------------------------------------------------- the step
def run_steps(z, cfg, st, flags, k0, k1, events=None):
    """Steps k0..k1-1 (t = k+1), rotating through the copies.  A step is one
    zero1_mta_step call (for the two-phase designs its reduce, finalize and
    update launches; the single launch when ONCHIP is asked for).  With
    events (events[i] = (start, end) pairs) a two-phase step is made as its two
    calls instead, zero1_mta_reduce + zero1_mta_update, so that the reduce
    kernel and the update kernel each stamp their own pair
    (zero1_time_next_launch: from the kernel's dispatch, no markers around
    it); the single launch gets stream markers around the whole call."""
    W, rank = st["W"], st["rank"]
    copies = st["copies"]
    two_phase = bool(flags & (z.STORE_G | z.RECOMPUTE_G))
    for k in range(k0, k1):
        c = copies[k % len(copies)]
        h = hp(cfg, k + 1)
        ev = events[k - k0] if events is not None else None
        if two_phase and not ev:
            z.mta_step(c.grads, c.begin, c.plan, h, c.rsd, W, rank, flags=flags, ws=c.ws)
        elif two_phase:
            z.time_next_launch(*ev[0])
            z.mta_reduce(c.grads, c.begin, c.plan, c.rsd[rank:rank + 1], flags=flags, ws=c.ws)
            z.time_next_launch(*ev[1])
            z.mta_update(c.grads, c.begin, c.plan, h, c.rsd, W, flags=flags, ws=c.ws)
        else:
            if ev:
                ev[0][0].record()
            z.mta_step(c.grads, c.begin, c.plan, h, c.rsd, W, rank, flags=flags, ws=c.ws)
            if ev:
                ev[0][1].record()


# ---------------------------------------------------------------------- CPU baseline
def cpu_baseline(cfg, S_total, begin, budget_s=12.0, max_steps=2000):
    """The oracle, as it stands, on the same rank's shard (a bounded sample):
    as many full steps as fit in about budget_s seconds of host time."""
    import numpy as np
    import oracle
    import synth

    W = cfg.W
    n = min(S_total, 16 * 1024 * 1024)     # at most 16M parameters of the shard
    grads = [synth.bf16(n, synth.grad_key(cfg.seed, 1, w), begin, cfg.sigma, cfg.outlier_pct) for w in range(W)]
    master = synth.f32(n, synth.master_key(cfg.seed), begin, cfg.master_sigma)
    mvd = np.uint16 if cfg.mv_bf16 else np.float32
    m, v = np.zeros(n, mvd), np.zeros(n, mvd)
    param = np.zeros(n, np.uint16)
    rs = np.zeros(W)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle.step(grads, master, m, v, param, hp(cfg, steps + 1), rs, cfg.rank % W)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= max_steps:
            break
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": n * steps / el, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full oracle steps (reduce, norm, clip, AdamW, bf16) on the first {n:,} "
                      f"parameters of the same rank's shard, W={W}, {el:.1f} s on {threads} threads",
            "cpu": cpu, "host_cpus": os.cpu_count()}


# ---------------------------------------------------------------------- PMC summary
def read_pmc_dir(d):
    """{kernel name: [per-dispatch counter values]} from a rocprofv3 --pmc output dir."""
    out = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True)
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
                val = row.get("Counter_Value") or row.get("Counter-Value")
                disp = row.get("Dispatch_Id") or row.get("Dispatch-Id") or str(len(out))
                if val is None:
                    continue
                out.setdefault(name, {}).setdefault(disp, 0.0)
                out[name][disp] += float(val)
    return {k: list(v.values()) for k, v in out.items()}


def summarize_pmc(fetch_dir, write_dir, out_path, kernel=UPDATE_KERNEL, also=()):
    """Median FETCH_SIZE / WRITE_SIZE per dispatch of `kernel`, scaled by what
    the same counters read for a torch.neg over CALIB_BYTES (a plain copy:
    CALIB_BYTES read, CALIB_BYTES written), appended to out_path; the same for
    each kernel whose name contains one of `also` (e.g. the step's reduce,
    named with its template arguments), as also_* lines."""
    fetch, write = read_pmc_dir(fetch_dir), read_pmc_dir(write_dir)

    def pick(d, key):
        for k, v in d.items():
            if key in k:
                return k, v
        raise SystemExit(f"no kernel matching {key!r} in {list(d)[:10]}")

    import statistics as stt
    kf, vf = pick(fetch, kernel)
    _, vw = pick(write, kernel)
    _, cf = pick(fetch, "neg_kernel")
    _, cw = pick(write, "neg_kernel")
    f_scale = (CALIB_BYTES / 1024.0) / stt.median(cf)
    w_scale = (CALIB_BYTES / 1024.0) / stt.median(cw)
    fb = stt.median(vf) * 1024 * f_scale
    wb = stt.median(vw) * 1024 * w_scale
    lines = [f"kernel_source_hash = {kernel_source_hash()}",
             f"dominant_kernel = {kernel}",
             f"# {kf[:110]}",
             f"# calibration: torch.neg over {CALIB_BYTES} B fp32 reads FETCH_SIZE {stt.median(cf):.1f} KiB "
             f"and WRITE_SIZE {stt.median(cw):.1f} KiB; scale fetch x{f_scale:.4f}, write x{w_scale:.4f}",
             f"# raw per dispatch (median of {len(vf)}): FETCH_SIZE {stt.median(vf):.1f} KiB, "
             f"WRITE_SIZE {stt.median(vw):.1f} KiB",
             f"dominant_fetch_bytes = {fb:.0f}",
             f"dominant_write_bytes = {wb:.0f}"]
    for name in also:
        ka, va = pick(fetch, name)
        _, wa = pick(write, name)
        lines += [f"also_kernel = {name}",
                  f"# raw per dispatch (median of {len(va)}): FETCH_SIZE {stt.median(va):.1f} KiB, "
                  f"WRITE_SIZE {stt.median(wa):.1f} KiB",
                  f"also_fetch_bytes = {stt.median(va) * 1024 * f_scale:.0f}",
                  f"also_write_bytes = {stt.median(wa) * 1024 * w_scale:.0f}"]
    with open(out_path, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_kt(kt_dir, out_path):
    """Per-kernel dispatch statistics from a rocprofv3 --kernel-trace output dir,
    split by grid size (the whole-shard reduce and the bucket reduces are the
    same kernel at different grids), appended to out_path."""
    import statistics as stt
    rows = {}
    for f in glob.glob(os.path.join(kt_dir, "**", "*kernel_trace*.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                short = name.replace("void ", "").replace("z1::(anonymous namespace)::", "").split("(")[0]
                grid = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                rows.setdefault((short, grid), []).append(dur)
    lines = [f"{'kernel':<48} | {'workgroups':>10} | {'calls':>5} | {'avg_us':>8} | {'median_us':>9} | "
             f"{'min_us':>8} | {'max_us':>8}"]
    for (short, grid), d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{short[:48]:<48} | {grid:>10} | {len(d):>5} | {sum(d) / len(d):>8.2f} | "
                     f"{stt.median(d):>9.2f} | {min(d):>8.2f} | {max(d):>8.2f}")
    with open(out_path, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_from_summary(path, kernel):
    """Counter bytes per launch of `kernel` from the committed summary, or None
    if the kernels changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = (s.strip() for s in line.split("=", 1))
            kv[k] = v
    if kv.get("kernel_source_hash") != kernel_source_hash() or kv.get("dominant_kernel") != kernel:
        return None
    try:
        return float(kv["dominant_fetch_bytes"]) + float(kv["dominant_write_bytes"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------- main
def bucketed_timing(torch, z, cfg, st, k0, steps, bucket_bytes=25_000_000):
    """The ZeRO-2-style flow on the same shard: the reduce runs per bucket (a
    25 MB bucket of the whole model's bf16 gradient is 25e6 / (2 W) of this
    rank's shard elements, rounded to whole 2048-element tiles), buckets in
    reverse order as backward would produce them; what is left after backward
    is the partials sum and the update.  Returns per step (ms): the GPU time of
    all bucket calls (stream markers around each call: its reduce and partial
    kernels, summed) and the time from the last bucket to the end of the
    update.  (Kernel-scoped events are not used here: on launches this short
    they lengthen the kernel they time by ~1.6 us.)"""
    W, rank, S = st["W"], st["rank"], st["S"]
    b = max(2048, bucket_bytes // (2 * W) // 2048 * 2048)
    ranges = [(lo, min(S, lo + b)) for lo in range(0, S, b)][::-1]
    nb = len(ranges)
    stream = torch.cuda.current_stream().cuda_stream
    calls = []
    for c in st["copies"]:
        if not hasattr(c, "parts"):
            c.parts = torch.zeros(nb, dtype=torch.float64, device=c.master.device)
        # addresses prepared once, so the timed loop is one C call per bucket
        calls.append([([g.data_ptr() + 2 * (c.begin + lo) for g in c.grads], lo, hi,
                       c.parts.data_ptr() + 8 * (nb - 1 - i)) for i, (lo, hi) in enumerate(ranges)])
    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()   # torch creates the event at its first record
        return e

    red_ms, crit_ms = [], []
    for k in range(k0, k0 + steps):
        ci = k % len(st["copies"])
        c = st["copies"][ci]
        ev = [event() for _ in range(2 * nb + 1)]
        torch.cuda.synchronize()
        for i, (gp, lo, hi, part) in enumerate(calls[ci]):
            ev[2 * i].record()
            z.mta_reduce_range(gp, c.plan, lo, hi, part, flags=z.STORE_G, ws=c.ws, stream=stream)
            ev[2 * i + 1].record()
        z.partials_sum(c.parts, nb, c.rsd[rank:rank + 1], stream=stream)
        z.mta_update(c.grads, c.begin, c.plan, hp(cfg, k + 1), c.rsd, W, flags=z.STORE_G, ws=c.ws, stream=stream)
        ev[2 * nb].record()
        torch.cuda.synchronize()
        red_ms.append(sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(nb)))
        crit_ms.append(ev[2 * nb - 1].elapsed_time(ev[2 * nb]))
    return dict(bucket_params=b, buckets=nb, reduce_ms=sum(red_ms) / steps,
                after_backward_ms=sum(crit_ms) / steps)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--design", choices=["auto", "onchip", "store", "recompute"], default="auto")
    ap.add_argument("--rotate", type=int, default=0, help="independent copies to rotate (0: auto)")
    ap.add_argument("--layout", choices=["arena", "packed"], default="arena",
                    help="arena: arrays placed by zero1_arena_plan; packed: one torch allocation each")
    ap.add_argument("--arena-size", choices=["fit", "all"], default="fit",
                    help="fit: the arena is as large as the plan; all: all free memory less 8 GB")
    ap.add_argument("--arena-offset-gib", type=float, default=0.0,
                    help="place the planned layout this far into the arena (tuning; needs --arena-size all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--pmc-also", action="append", default=[], metavar="KERNEL",
                    help="with --summarize-pmc: also summarize kernels whose name contains this")
    ap.add_argument("--summarize-kt", nargs=2, metavar=("KT_DIR", "OUT"))
    a = ap.parse_args()

    if a.summarize_pmc:
        summarize_pmc(*a.summarize_pmc, also=a.pmc_also)
        return 0
    if a.summarize_kt:
        summarize_kt(*a.summarize_kt)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one rank's step on ONE GPU; --gpus {a.gpus} (WORLD_SIZE={world}) is not "
              "supported: the library runs one rank's step; several GPUs would each run it on their own shard "
              "with the exchanges around it, which is not part of this library",
              file=sys.stderr)
        return 2

    import torch
    import zero_sharded_mixed_zero1_amd as z
    from synth.workloads import configs

    cfg = configs()[a.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flags = {"auto": 0, "onchip": z.ONCHIP, "store": z.STORE_G, "recompute": z.RECOMPUTE_G}[a.design]
    store_g = bool(flags & z.STORE_G) or (not (flags & (z.RECOMPUTE_G | z.ONCHIP)) and cfg.W > 4)
    per_copy = cfg.S * (2 * cfg.W + 26 + (4 if store_g else 0))
    n_copies = a.rotate or (2 if per_copy < (1 << 30) else 1)
    st = setup(torch, cfg, flags, n_copies, dev, a.layout, a.arena_size == "all",
               int(a.arena_offset_gib * (1 << 30)))
    S, W = st["S"], st["W"]
    c0 = st["copies"][0]
    design = z.mta_design(c0.grads, c0.begin, c0.plan, flags)
    if design == 0:
        print(f"design {a.design} is not possible for {a.config}", file=sys.stderr)
        return 2
    flags = (flags & ~(z.ONCHIP | z.STORE_G | z.RECOMPUTE_G)) | design   # run the resolved design explicitly
    design_name = {z.ONCHIP: "onchip", z.STORE_G: "store_g", z.RECOMPUTE_G: "recompute_g"}[design]

    if a.pmc_run:
        run_steps(z, cfg, st, flags, 0, 4)
        x = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print("pmc run done", flush=True)
        return 0

    run_steps(z, cfg, st, flags, 0, a.warmup)
    torch.cuda.synchronize()
    # the timed region: exactly K steps back to back, bracketed by synchronizations
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    run_steps(z, cfg, st, flags, a.warmup, a.warmup + a.steps)
    g1.record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    gpu_ms_per_step = g0.elapsed_time(g1) / a.steps
    # each kernel's own duration: the same K steps again, the reduce and the
    # update of each stamped by their own dispatches (HIP events; the single
    # launch is bracketed by stream markers on the stream it runs on)
    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()   # torch creates the event at its first record
        return e

    events = [((event(), event()), (event(), event())) for _ in range(a.steps)]
    torch.cuda.synchronize()
    run_steps(z, cfg, st, flags, a.warmup + a.steps, a.warmup + 2 * a.steps, events)
    torch.cuda.synchronize()
    two_phase = bool(flags & (z.STORE_G | z.RECOMPUTE_G))
    kern_ms = [e[1 if two_phase else 0][0].elapsed_time(e[1 if two_phase else 0][1]) for e in events]
    red_ms = [e[0][0].elapsed_time(e[0][1]) for e in events] if two_phase else None
    ms_per_step = el * 1e3 / a.steps
    value = S / (ms_per_step * 1e-3)
    bpp = cfg.bytes_per_param
    kern_avg = sum(kern_ms) / len(kern_ms)
    # algorithmic bytes per launch of the dominant kernel: the whole step
    # (2W+26 B/param) for the single launch; master/m/v read+write and the
    # bf16 write (26 B/param, 18 with bf16 m,v) for the two-phase update
    kern_bytes = ((18 if cfg.mv_bf16 else 26) if two_phase else bpp) * S
    kern_name = UPDATE_KERNEL if two_phase else ONCHIP_KERNEL
    achieved = kern_bytes / (kern_avg * 1e-3) / 1e9
    traffic = traffic_from_summary(PMC_SUMMARY, kern_name) if (a.config == "C2" and a.design == "auto") else None
    out = {
        "metric": "params updated/s and achieved HBM GB/s (% of peak) per fused ZeRO-1 step",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64 Irwin-Hall gradients and masters; tensor shapes only, no weights)",
        "config": {
            "workload": cfg.workload,
            "W": W, "rank": st["rank"], "shard_params": S, "pieces": st["pieces"],
            "bytes_per_param": bpp, "design": design_name,
            "rotated_copies": n_copies, "m_v": "bf16" if cfg.mv_bf16 else "fp32",
            "memory_layout": st["info"],
        },
        "algorithmic_GBps": value * bpp / 1e9,
        "pct_of_peak_hbm": 100.0 * value * bpp / 1e9 / PEAK_HBM_GBS,
        "gpu_ms_per_step": gpu_ms_per_step,
        "kernel_ms": kern_avg,
        "reduce_kernel_ms": sum(red_ms) / len(red_ms) if red_ms else None,
        "roofline": {"bound": "hbm", "kernel": kern_name, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": kern_bytes},
    }
    if red_ms:
        # both kernels of the two-phase step: bytes the step's algorithm needs
        # and bytes the design moves (+ the fp32 g written and re-read, or the
        # slices re-read), over each kernel's own time
        red_avg = sum(red_ms) / len(red_ms)
        store_g = bool(flags & z.STORE_G)
        red_alg, red_mv = 2 * W * S, (2 * W + (4 if store_g else 0)) * S
        upd_mv = kern_bytes + (4 if store_g else 2 * W) * S
        out["kernels"] = {
            "reduce": {"ms": red_avg, "algorithmic_bytes": red_alg, "moved_bytes": red_mv,
                       "algorithmic_GBps": red_alg / (red_avg * 1e-3) / 1e9,
                       "moved_GBps": red_mv / (red_avg * 1e-3) / 1e9},
            "update": {"ms": kern_avg, "algorithmic_bytes": kern_bytes, "moved_bytes": upd_mv,
                       "algorithmic_GBps": achieved, "moved_GBps": upd_mv / (kern_avg * 1e-3) / 1e9},
        }
    if flags & z.STORE_G:
        out["bucketed"] = bucketed_timing(torch, z, cfg, st, a.warmup + 2 * a.steps, min(a.steps, 50))
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, S, st["begin"])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
