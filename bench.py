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

Prints ONE JSON line.  Metric: shard parameters updated per second; the
algorithmic HBM traffic is (2W+26) bytes per parameter (W bf16 gradient reads,
fp32 master/m/v read + write, bf16 parameter write).

Modes:
  python bench.py [--steps K] [--warmup W] [--config C2]    the benchmark line
  python bench.py --pmc-run                                   short run for rocprofv3 --pmc
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR OUT     counter summary for profiles/
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
REDUCE_KERNEL = "reduce_kernel"
CALIB_BYTES = 1 << 30          # the plain copy used to scale the PMC byte counters
PMC_SUMMARY = os.path.join(ROOT, "profiles", "adamw_mta_gpt2small_w8_pmc.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in ("zero_sharded_mixed_zero1_amd/csrc/kernels.hip", "zero_sharded_mixed_zero1_amd/csrc/internal.h",
              "zero_sharded_mixed_zero1_amd/csrc/api.cpp"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------- setup
class Copy:
    """One independent copy of everything a step touches (rotated through so
    that consecutive steps do not find each other's data in the 256 MB MALL)."""


def setup(torch, cfg, design_flags, n_copies, dev):
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
    copies = []
    for c in range(n_copies):
        cp = Copy()
        if cfg.all_replicas_resident:
            # every replica's full flat gradient is resident; the step reads rank's slice
            cp.full = [torch.empty(N, dtype=torch.int16, device=dev) for _ in range(W)]
            for w, t in enumerate(cp.full):
                synth.fill_bf16_(t, synth.grad_key(cfg.seed, 1, w), 0, cfg.sigma, cfg.outlier_pct)
            cp.grads = cp.full
            cp.begin = begin
        else:
            # only this rank's W slices exist (their global flat indices start at begin)
            cp.grads = [torch.empty(S, dtype=torch.int16, device=dev) for _ in range(W)]
            for w, t in enumerate(cp.grads):
                synth.fill_bf16_(t, synth.grad_key(cfg.seed, 1, w), begin, cfg.sigma, cfg.outlier_pct)
            cp.begin = 0
        cp.master = torch.empty(S, dtype=torch.float32, device=dev)
        synth.fill_f32_(cp.master, synth.master_key(cfg.seed), begin, cfg.master_sigma)
        mvdt = torch.int16 if cfg.mv_bf16 else torch.float32
        cp.m = torch.zeros(S, dtype=mvdt, device=dev)
        cp.v = torch.zeros(S, dtype=mvdt, device=dev)
        # the whole model's bf16 parameters, one buffer per tensor list (pieces point inside)
        first, last = pieces_l[0][0], pieces_l[-1][0]
        lo, hi = offsets[first], offsets[last + 1]
        cp.params = torch.zeros(hi - lo, dtype=torch.int16, device=dev)
        pieces = [(n, so, cp.params[offsets[ti] - lo + off:], cp.master[so:], cp.m[so:], cp.v[so:])
                  for ti, off, so, n in pieces_l]
        cp.table = torch.empty(max(256, z.mta_table_bytes(pieces)), dtype=torch.uint8, device=dev)
        cp.plan = z.mta_plan(pieces, cp.table, flags=z.MV_BF16 if cfg.mv_bf16 else 0)
        cp.ws = torch.empty(z.mta_workspace_bytes(cp.plan, W, design_flags), dtype=torch.uint8, device=dev)
        cp.rsd = torch.zeros(W, dtype=torch.float64, device=dev)
        copies.append(cp)
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
    return dict(W=W, rank=rank, N=N, S=S, begin=begin, pieces=len(pieces_l), copies=copies)


def hp(cfg, t):
    return cfg.hparams(t)


# ---------------------------------------------------------------------- the step
def run_steps(torch, z, cfg, st, flags, k0, k1, events=None):
    """Steps k0..k1-1 (t = k+1), rotating through the copies."""
    W, rank = st["W"], st["rank"]
    copies = st["copies"]
    for k in range(k0, k1):
        c = copies[k % len(copies)]
        h = hp(cfg, k + 1)
        if events is not None:
            events[k - k0][0].record()
        z.mta_reduce(c.grads, c.begin, c.plan, c.rsd[rank:rank + 1], flags=flags, ws=c.ws)
        if events is not None:
            events[k - k0][1].record()
        z.mta_update(c.grads, c.begin, c.plan, h, c.rsd, W, flags=flags, ws=c.ws)
        if events is not None:
            events[k - k0][2].record()


# ---------------------------------------------------------------------- CPU baseline
def cpu_baseline(cfg, S_total, begin, budget_s=12.0):
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
        if el >= budget_s or steps >= 200:
            break
    return {"value": n * steps / el, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full oracle steps (reduce, norm, clip, AdamW, bf16) on the first {n:,} "
                      f"parameters of the same rank's shard, W={W}, {el:.1f} s on {threads} threads"}


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


def summarize_pmc(fetch_dir, write_dir, out_path):
    fetch, write = read_pmc_dir(fetch_dir), read_pmc_dir(write_dir)

    def pick(d, key):
        for k, v in d.items():
            if key in k:
                return k, v
        raise SystemExit(f"no kernel matching {key!r} in {list(d)[:10]}")

    import statistics as stt
    res = {}
    for tag, key in (("update", UPDATE_KERNEL), ("reduce", REDUCE_KERNEL), ("calib", "neg")):
        kf, vf = pick(fetch, key if tag != "calib" else "neg")
        kw, vw = pick(write, key if tag != "calib" else "neg")
        res[tag] = dict(kernel=kf, fetch_kib=stt.median(vf), write_kib=stt.median(vw), n=len(vf))
    cal = res["calib"]
    f_scale = (CALIB_BYTES / 1024.0) / cal["fetch_kib"]
    w_scale = (CALIB_BYTES / 1024.0) / cal["write_kib"]
    lines = [f"kernel_source_hash = {kernel_source_hash()}",
             f"calibration: torch.neg of {CALIB_BYTES} bytes fp32 -> FETCH_SIZE {cal['fetch_kib']:.1f} KiB, "
             f"WRITE_SIZE {cal['write_kib']:.1f} KiB; scale fetch {f_scale:.4f}, write {w_scale:.4f}"]
    for tag in ("update", "reduce"):
        r = res[tag]
        fb = r["fetch_kib"] * 1024 * f_scale
        wb = r["write_kib"] * 1024 * w_scale
        lines.append(f"{tag}: {r['kernel'][:90]}")
        lines.append(f"{tag}_fetch_bytes = {fb:.0f}")
        lines.append(f"{tag}_write_bytes = {wb:.0f}")
        lines.append(f"{tag}_dispatches = {r['n']}")
    with open(out_path, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_from_summary(path):
    """Counter bytes per update launch from the committed summary, or None if
    the kernels changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = (s.strip() for s in line.split("=", 1))
            kv[k] = v
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["update_fetch_bytes"]) + float(kv["update_write_bytes"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--design", choices=["auto", "store", "recompute"], default="auto")
    ap.add_argument("--rotate", type=int, default=0, help="independent copies to rotate (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    a = ap.parse_args()

    if a.summarize_pmc:
        summarize_pmc(*a.summarize_pmc)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one rank's step on ONE GPU; --gpus {a.gpus} (WORLD_SIZE={world}) is not "
              "supported: this build has no multi-GPU path (the step shards by construction; see DESIGN.md)",
              file=sys.stderr)
        return 2

    import torch
    import zero_sharded_mixed_zero1_amd as z
    from synth.workloads import configs

    cfg = configs()[a.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flags = {"auto": 0, "store": z.STORE_G, "recompute": z.RECOMPUTE_G}[a.design]
    store_g = bool(flags & z.STORE_G) or (not (flags & z.RECOMPUTE_G) and cfg.W > 4)
    per_copy = cfg.S * (2 * cfg.W + 26 + (4 if store_g else 0))
    n_copies = a.rotate or (2 if per_copy < (1 << 30) else 1)
    st = setup(torch, cfg, flags, n_copies, dev)
    S, W = st["S"], st["W"]

    if a.pmc_run:
        run_steps(torch, z, cfg, st, flags, 0, 4)
        x = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print("pmc run done", flush=True)
        return 0

    run_steps(torch, z, cfg, st, flags, 0, a.warmup)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(torch, z, cfg, st, flags, a.warmup, a.warmup + a.steps, events)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    red_ms = [e[0].elapsed_time(e[1]) for e in events]
    upd_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = el * 1e3 / a.steps
    value = S / (ms_per_step * 1e-3)
    bpp = cfg.bytes_per_param
    upd_avg = sum(upd_ms) / len(upd_ms)
    red_avg = sum(red_ms) / len(red_ms)
    upd_bytes = (18 if cfg.mv_bf16 else 26) * S          # master/m/v read+write + bf16 param write
    achieved = upd_bytes / (upd_avg * 1e-3) / 1e9
    traffic = traffic_from_summary(PMC_SUMMARY) if a.config == "C2" and n_copies == 2 and a.design == "auto" else None
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    c = st["copies"][0]
    z.mta_update(c.grads, c.begin, c.plan, hp(cfg, 1), c.rsd, W, flags=flags, info_out=info, ws=c.ws)
    torch.cuda.synchronize()
    ni = info.cpu().numpy()
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
            "bytes_per_param": bpp, "design": "store_g" if store_g else "recompute_g",
            "rotated_copies": n_copies, "m_v": "bf16" if cfg.mv_bf16 else "fp32",
            "global_norm": float(ni[1]), "clipped": bool(ni[2:4].view("int32")[1]),
        },
        "algorithmic_GBps": value * bpp / 1e9,
        "pct_of_peak_hbm": 100.0 * value * bpp / 1e9 / PEAK_HBM_GBS,
        "kernels_ms": {"reduce_phase(reduce+finalize)": red_avg, "update(adamw_mta)": upd_avg},
        "roofline": {"bound": "hbm", "kernel": UPDATE_KERNEL, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": upd_bytes},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, S, st["begin"])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
