#!/usr/bin/env python3
"""Benchmark: one data-parallel rank's fused ZeRO-1 optimizer step on one MI355X.

A step is the whole hot path for one rank's shard: reduce the W replicas' bf16
gradient slices (fp32, rank order, / W), this rank's fp64 sum of squares, the
global-norm clip, AdamW (update, then decay) on the fp32 master/m/v, and the
bf16 parameter write-back over the ragged per-tensor list (multi-tensor apply).

Headline workload: the full AdamW step of a dense 7e9-parameter model at W=1
(no reduction; fp32 master, m, v: 16 B/param of state, 28 B/param moved per
step), the largest configuration that fits one GPU.  The same line carries
`per_config`: the other workloads (flat 2^20 W=4, GPT-2 small W=8, dense 7.5e9
W=64, Llama-7B W=8, the 7e9 step with bf16 m, v), each timed the same way.
All inputs are synthetic (seeded) and resident in HBM before any timed region.
For the workloads whose other ranks' gradients are not resident, the other
ranks' partial sums of squares are 0 (the norm is this shard's own).

Every workload is measured in two memory layouts: "arena" (every array of the
step in one allocation laid out by zero1_arena_plan: the update's five streams
40 GiB apart) and "packed" (one torch allocation per array).  The headline
`value` is the arena figure; the packed one is reported beside it.

Per kernel the line gives the algorithmic bytes over its own duration (HIP
events stamped by the kernel's dispatch), the bytes the design moves, and a
same-traffic calibration: the time of a kernel that moves exactly the same
streams with the same access pattern and placement and computes nothing
(libzero1_calib.so).  Secondary passes in each layout: the step's kernels with
4 GiB of other tensors written before every step (in the arena's gaps, or a
separate tensor), and, for the workloads that rotate copies, the same steps on
one copy (MALL-warm).

Prints ONE JSON line.  Metric: shard parameters updated per second; the
algorithmic HBM traffic is (2W+26) bytes per parameter (W bf16 gradient reads,
fp32 master/m/v read + write, bf16 parameter write; 2W+18 with bf16 m, v).

Modes:
  python bench.py [--steps K] [--warmup W]                     the benchmark line
  python bench.py --config C4 [--layout arena] --no-per-config one workload only
  python bench.py --calibrate                                  plain read/write/copy rates, the step's
                                                               mixes, spacing, cache-policy and
                                                               placement sweeps
  python bench.py --pmc-run --config C                         short run for rocprofv3 --pmc
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR OUT      counter summary for profiles/
  python bench.py --summarize-kt KT_DIR OUT                    kernel-trace summary for profiles/
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import gc
import glob
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
UPDATE_KERNEL = "adamw_mta_kernel"
REDUCE_KERNEL = "reduce_kernel"
CALIB_BYTES = 1 << 30          # the plain copy used to scale the PMC byte counters
HEADLINE = "C5a"
PER_CONFIG = ("C1", "C2", "C3", "C4", "C5b")
# profile summaries are named for the workload they cover
WORKLOAD_TAG = {"C1": "flat1m_w4", "C2": "gpt2small_w8", "C3": "dense7p5b_w64", "C4": "llama7b_w8",
                "C5a": "dense7b_w1", "C5b": "dense7b_w1_bf16mv"}
# timed steps per layout of the small workloads (their steps take microseconds)
MIN_STEPS = {"C1": 400, "C2": 200}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


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


def pmc_summary_path(name):
    return os.path.join(ROOT, "profiles", f"zero1_step_{WORKLOAD_TAG[name]}_pmc.txt")


# ---------------------------------------------------------------------- calibration kernels
_cal = None


def cal_lib():
    global _cal
    if _cal is None:
        path = os.path.join(ROOT, "zero_sharded_mixed_zero1_amd", "libzero1_calib.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.zcal_stream.argtypes = [P, P, P, i32, P, P, P, i32, i64, i32, i32, i32, i32, i32, P, P]
        L.zcal_stream.restype = i32
        L.zcal_policy_mix.argtypes = [i32, i32, P, P, P, P, P, i64, i32, i32, P]
        L.zcal_policy_mix.restype = i32
        _cal = L
    return _cal


def zcal_stream(rd, wr, n_tiles, grid, split, sink, stream, tiles_in_flight=1, wide=0, contig=0):
    """One calibration pass.  rd: [(device address, bytes per element, plain
    loads?)]; wr: [(device address, bytes per element, sc1 stores?)]; every
    stream must hold n_tiles * 2048 elements from its address."""
    R, Wn = len(rd), len(wr)

    def arr(t, vals):
        return (t * max(len(vals), 1))(*vals)

    st = cal_lib().zcal_stream(arr(ctypes.c_void_p, [x[0] for x in rd]), arr(ctypes.c_int, [x[1] for x in rd]),
                               arr(ctypes.c_int, [int(x[2]) for x in rd]), R,
                               arr(ctypes.c_void_p, [x[0] for x in wr]), arr(ctypes.c_int, [x[1] for x in wr]),
                               arr(ctypes.c_int, [int(x[2]) for x in wr]), Wn,
                               n_tiles, tiles_in_flight, wide, contig, grid, split, sink, stream)
    if st != 0:
        raise RuntimeError(f"zcal_stream failed with status {st}")


def zcal_policy_mix(rd_policy, wr_policy, g, p, m, v, out, n_tiles, grid, split, stream):
    """One pass of the update's stream mix with explicit cache-policy bits
    (1 sc0, 2 nt, 16 sc1) on its loads and stores."""
    st = cal_lib().zcal_policy_mix(rd_policy, wr_policy, g, p, m, v, out, n_tiles, grid, split, stream)
    if st != 0:
        raise RuntimeError(f"zcal_policy_mix failed with status {st}")


def best_calibration(torch, rd, wr, n_tiles, grid, split, sink, stream, reps=5):
    """The fastest calibration pass over U (tiles whose loads are issued
    together) in {1, 2, 4, 8} with at most eight (tile, stream) loads in
    flight: (ms, U)."""
    best = None
    for U in (1, 2, 4, 8):
        if U > 1 and U * max(len(rd), 1) > 8:
            continue
        fn = lambda: zcal_stream(rd, wr, n_tiles, grid, split, sink, stream, U)  # noqa: E731
        fn()
        torch.cuda.synchronize()
        ms = timed_passes(torch, fn, reps)
        if best is None or ms < best[0]:
            best = (ms, U)
    return best


def timed_passes(torch, fn, reps):
    """Median duration (ms) of fn() over reps launches, each between HIP events
    on torch's current stream (the stream fn launches on)."""
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return statistics.median(out)


def launch_shape(units, cus, per_cu, big_split):
    """The library's grid for a pass over `units` tiles (internal grid_for):
    per_cu > 0 caps the grid at per_cu * CUs; a multiple of 8."""
    cap = min(cus * per_cu if per_cu > 0 else units, 8192)
    n = min(units, cap)
    if n > 8:
        n = (n + 7) // 8 * 8
    n = max(n, 1)
    return n, (8 if big_split(units, n) else 1)


# ---------------------------------------------------------------------- setup
class Copy:
    """One independent copy of everything a step touches (rotated through so
    that consecutive steps do not find each other's data in the 256 MB MALL)."""


def setup(torch, cfg, design_flags, n_copies, dev, layout="arena"):
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
        arena = torch.empty(total, dtype=torch.uint8, device=dev)
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
        cp.shard_params = cp.params[begin - p_lo:begin - p_lo + S]
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
    spans = sorted(spans) if arena is not None else []
    if arena is not None:   # no two arrays of any copy overlap (checked before any step runs)
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
    return dict(W=W, rank=rank, N=N, S=S, begin=begin, pieces=len(pieces_l), copies=copies, info=info,
                arena=arena, spans=spans)


# ---------------------------------------------------------------------- the step
def run_steps(z, cfg, st, flags, k0, k1, events=None):
    """Steps k0..k1-1 (t = k+1), rotating through the copies.  A step is one
    zero1_mta_step call (its reduce, finalize and update launches).  With
    events (events[i] = (start, end) pairs) each step is made as its two
    calls instead, zero1_mta_reduce + zero1_mta_update, so that the reduce
    kernel and the update kernel each stamp their own pair
    (zero1_time_next_launch: from the kernel's dispatch, no markers around it)."""
    W, rank = st["W"], st["rank"]
    copies = st["copies"]
    for k in range(k0, k1):
        c = copies[k % len(copies)]
        h = cfg.hparams(k + 1)
        if events is None:
            z.mta_step(c.grads, c.begin, c.plan, h, c.rsd, W, rank, flags=flags, ws=c.ws)
        else:
            ev = events[k - k0]
            z.time_next_launch(*ev[0])
            z.mta_reduce(c.grads, c.begin, c.plan, c.rsd[rank:rank + 1], flags=flags, ws=c.ws)
            z.time_next_launch(*ev[1])
            z.mta_update(c.grads, c.begin, c.plan, h, c.rsd, W, flags=flags, ws=c.ws)


def calibrated(torch, z, cfg, st, store_g, cus):
    """Same-traffic calibration of the two kernels of the step: the same
    streams (copy 0's arrays, at their addresses), moved with the same access
    pattern and launch shape by a kernel that computes nothing -- what HBM
    delivers for that traffic, a reference for the step kernels (which run a
    little faster than this generic kernel).  Run after the timed passes (it
    overwrites the arrays)."""
    W, S = st["W"], st["S"]
    c = st["copies"][0]
    mvb = 2 if cfg.mv_bf16 else 4

    def al(addr):            # first 16-byte aligned address at or after addr
        return (addr + 15) // 16 * 16

    n_tiles = max(0, (S - 8) // 2048)
    if n_tiles == 0:
        return None
    grads = [al(g.data_ptr() + 2 * c.begin) for g in c.grads]
    state = [(al(c.master.data_ptr()), 4), (al(c.m.data_ptr()), mvb), (al(c.v.data_ptr()), mvb)]
    state_rd = [(a, b, False) for a, b in state]
    state_wr = [(a, b, False) for a, b in state] + [(al(c.shard_params.data_ptr()), 2, False)]
    if store_g:
        # the g region of the workspace; a g that fits the MALL is stored with
        # sc1 and read back with plain loads, as the step kernels do
        g = al(c.ws.data_ptr() + 256 + 8 * 8192)
        small = 4 * S <= (128 << 20)
        red_rd, red_wr = [(a, 2, False) for a in grads], [(g, 4, small)]
        upd_rd = [(g, 4, small)] + state_rd
    else:
        red_rd, red_wr = [(a, 2, False) for a in grads], []
        upd_rd = [(a, 2, False) for a in grads] + state_rd
    sink = torch.zeros(8192, dtype=torch.int32, device=c.master.device)
    stream = torch.cuda.current_stream().cuda_stream
    # the library's reduce grid: 8 workgroups per CU, 6 for the sum-of-squares
    # pass over one to four slices (its few-slice kernel)
    rg, rs = launch_shape(n_tiles, cus, 8 if store_g else 6, lambda u, n: u >= 16 * n)
    ug, us = launch_shape(n_tiles, cus, 8 if n_tiles > 8192 else 0, lambda u, n: u > 8192)
    out = {}
    passes = (("reduce", red_rd, red_wr, rg, rs), ("update", upd_rd, state_wr, ug, us))
    for name, rd, wr, grid, split in passes:
        ms, U = best_calibration(torch, rd, wr, n_tiles, grid, split, sink.data_ptr(), stream)
        nbytes = n_tiles * 2048 * (sum(x[1] for x in rd) + sum(x[1] for x in wr))
        out[name] = {"ms": ms, "bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
                     "shard_ms": ms * S / (n_tiles * 2048), "tiles_in_flight": U}

    # the two passes back to back, as the step runs them (the update finds
    # in the MALL what the reduce's sc1 stores left there)
    def pair():
        for name, rd, wr, grid, split in passes:
            zcal_stream(rd, wr, n_tiles, grid, split, sink.data_ptr(), stream, out[name]["tiles_in_flight"])

    out["step_shard_ms"] = timed_passes(torch, pair, 5) * S / (n_tiles * 2048)
    return out


def measure(torch, z, cfg, layout, steps, warmup, dev, bucketed=False):
    """One workload in one layout: warmup, K timed steps, K kernel-timed steps,
    the same-traffic calibration (and, for the store-g design, the bucketed flow)."""
    W = cfg.W
    store_g = W > 4
    # copies rotated so that a step never finds the previous steps' data in
    # the 256 MB MALL: at least 512 MiB of other traffic between two uses of
    # one copy (bytes a step touches per copy: the design's byte count)
    per_copy = cfg.S * (2 * W + 26 + (4 if store_g else 0))
    n_copies = 1 if per_copy >= (1 << 30) else min(64, max(2, -(-(512 << 20) // per_copy) + 1))
    design = z.STORE_G if store_g else z.RECOMPUTE_G
    gc.collect()
    st = setup(torch, cfg, design, n_copies, dev, layout)
    S = st["S"]
    c0 = st["copies"][0]
    assert z.mta_design(c0.grads, c0.begin, c0.plan, 0) == design
    run_steps(z, cfg, st, design, 0, warmup)
    torch.cuda.synchronize()
    # no garbage collection inside the timed passes: a full collection (tens
    # of ms with torch loaded) would land in the middle of a step
    gc.collect()
    gc.disable()
    # the timed region: exactly K steps back to back, bracketed by synchronizations
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    run_steps(z, cfg, st, design, warmup, warmup + steps)
    g1.record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    gpu_ms = g0.elapsed_time(g1) / steps

    # each kernel's own duration: the same K steps again, each as its two
    # calls, with the reduce and the update stamped by their own dispatches
    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()   # torch creates the event at its first record
        return e

    events = [((event(), event()), (event(), event())) for _ in range(steps)]
    torch.cuda.synchronize()
    run_steps(z, cfg, st, design, warmup + steps, warmup + 2 * steps, events)
    torch.cuda.synchronize()
    gc.enable()
    upd_t = [e[1][0].elapsed_time(e[1][1]) for e in events]
    red_t = [e[0][0].elapsed_time(e[0][1]) for e in events]
    upd_ms, red_ms = statistics.fmean(upd_t), statistics.fmean(red_t)
    ms = el * 1e3 / steps
    bpp = cfg.bytes_per_param
    fixed = 18 if cfg.mv_bf16 else 26
    # algorithmic bytes per launch: store-g -- the reduce does the 2W gradient
    # reads, the update the fixed bytes; recompute -- the update does every
    # algorithmic access (it reads the slices, the state, writes the state and
    # the parameters) and the sum-of-squares pass is design overhead
    if store_g:
        red_alg, red_mv = 2 * W * S, (2 * W + 4) * S
        upd_alg, upd_mv = fixed * S, (fixed + 4) * S
    else:
        red_alg, red_mv = 0, 2 * W * S
        upd_alg, upd_mv = (2 * W + fixed) * S, (2 * W + fixed) * S
    res = {
        "layout": st["info"], "steps": steps, "warmup": warmup, "rotated_copies": n_copies,
        "ms_per_step": ms, "gpu_ms_per_step": gpu_ms, "params_per_s": S / (ms * 1e-3),
        "algorithmic_GBps": bpp * S / (ms * 1e-3) / 1e9,
        "pct_of_peak_hbm": 100.0 * bpp * S / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "moved_bytes_per_step": red_mv + upd_mv,
        "kernels": {
            "reduce": {"ms": red_ms, "algorithmic_bytes": red_alg, "moved_bytes": red_mv,
                       "algorithmic_GBps": red_alg / (red_ms * 1e-3) / 1e9,
                       "moved_GBps": red_mv / (red_ms * 1e-3) / 1e9},
            "update": {"ms": upd_ms, "algorithmic_bytes": upd_alg, "moved_bytes": upd_mv,
                       "algorithmic_GBps": upd_alg / (upd_ms * 1e-3) / 1e9,
                       "moved_GBps": upd_mv / (upd_ms * 1e-3) / 1e9},
        },
    }
    for k, t in (("reduce", red_t), ("update", upd_t)):
        kk = res["kernels"][k]
        kk["ms_median"], kk["ms_min"] = statistics.median(t), min(t)
        kk["frac_of_peak"] = kk["algorithmic_GBps"] / PEAK_HBM_GBS
        kk["traffic"] = traffic_from_summary(pmc_summary_path(cfg.name), k) if layout == "arena" else None
    if bucketed and store_g:
        res["bucketed"] = bucketed_timing(torch, z, cfg, st, warmup + 2 * steps, min(steps, 50))
        gc.collect()
        gc.disable()
        res["bucketed"]["with_backward_gemms"] = bucketed_overlap(torch, z, cfg, st, warmup + 2 * steps + 60)
        gc.enable()
    if ms < 0.2:   # launch-bound sizes: the same step replayed from a captured graph
        gc.collect()
        gc.disable()
        res["graph"] = graph_timing(torch, z, cfg, st, design, warmup + 2 * steps + 100)
        gc.enable()
    if n_copies > 1:
        # secondary figure: the same K steps on copy 0 alone, so that each step
        # finds what the previous one left in the MALL
        gc.collect()
        gc.disable()
        warm = dict(st, copies=st["copies"][:1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(z, cfg, warm, design, warmup + 2 * steps, warmup + 3 * steps)
        torch.cuda.synchronize()
        res["mall_warm_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
        gc.enable()
    gc.collect()
    gc.disable()
    res["other_tensors"] = other_tensors(torch, z, cfg, st, design, warmup + 2 * steps + 300, steps, red_ms, upd_ms)
    gc.enable()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    cal = calibrated(torch, z, cfg, st, store_g, cus)
    if cal:
        for k in ("reduce", "update"):
            kk = res["kernels"][k]
            kk["calibrated_ms"] = cal[k]["shard_ms"]
            kk["calibrated_moved_GBps"] = cal[k]["GBps"]
            kk["calibrated_over_kernel"] = cal[k]["shard_ms"] / kk["ms"]
            kk["calibrated_tiles_in_flight"] = cal[k]["tiles_in_flight"]
        res["calibrated_ms_per_step"] = cal["step_shard_ms"]
    del st, c0
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def arena_gaps(st, min_bytes=64 << 20):
    """[a, b) byte ranges of the arena that no array of the step occupies
    (the gaps between the spaced arrays), at least min_bytes each."""
    total, pos, gaps = st["arena"].numel(), 0, []
    for a, b in st["spans"]:
        if a - pos >= min_bytes:
            gaps.append((pos, a))
        pos = max(pos, b)
    if total - pos >= min_bytes:
        gaps.append((pos, total))
    return gaps


OTHER_BYTES_PER_STEP = 4 << 30   # other tensors' writes between two steps


def other_tensors(torch, z, cfg, st, design, k0, steps, idle_red_ms, idle_upd_ms):
    """The step inside a training process whose other tensors are written
    between two optimizer steps: 4 GiB of writes (1 GiB fills) before each
    step -- in the arena layout into its gaps, every gap byte written once
    first (the gaps hold the other tensors); with one allocation per array into
    one separate 1 GiB tensor -- and the step's two kernels timed by their own
    dispatches, as in the idle passes."""
    dev = st["copies"][0].master.device
    if st["arena"] is not None:
        gaps = arena_gaps(st)
        if not gaps:
            return None
        views = [st["arena"][a:b] for a, b in gaps]
        for v in views:
            v.fill_(0x5A)
        where = f"the arena's {len(gaps)} gaps ({sum(b - a for a, b in gaps)} B, every byte written once first)"
    else:
        views = [torch.empty(1 << 30, dtype=torch.uint8, device=dev)]
        where = "one separate 1 GiB tensor"
    torch.cuda.synchronize()

    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    events = [((event(), event()), (event(), event())) for _ in range(steps)]
    fills = OTHER_BYTES_PER_STEP // (1 << 30)
    written = 0
    torch.cuda.synchronize()
    for i in range(steps):
        for j in range(fills):
            v = views[(i * fills + j) % len(views)]
            n = min(1 << 30, v.numel())
            o = ((i * fills + j) * n) % (v.numel() - n + 1)
            v[o:o + n].fill_((i + j) & 0xFF)
            written += n
        run_steps(z, cfg, st, design, k0 + i, k0 + i + 1, [events[i]])
    torch.cuda.synchronize()
    red = statistics.fmean(e[0][0].elapsed_time(e[0][1]) for e in events)
    upd = statistics.fmean(e[1][0].elapsed_time(e[1][1]) for e in events)
    del views
    return {"where": where, "written_per_step_bytes": written // steps, "reduce_ms": red, "update_ms": upd,
            "kernels_ms": red + upd, "over_idle": (red + upd) / (idle_red_ms + idle_upd_ms)}


# ---------------------------------------------------------------------- CPU baseline
CPU_SAMPLE = {"C1": None, "C2": None, "C3": 1 << 20, "C4": 1 << 22, "C5a": 1 << 23, "C5b": 1 << 23}


def cpu_model():
    """The host CPU as lscpu describes it: model name, family / model /
    stepping, sockets x cores x threads, L3 size, hypervisor (a virtual
    machine may report only a generic model name)."""
    fields = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    name = fields.get("Model name")
    if not name:
        try:
            with open("/proc/cpuinfo") as f:
                name = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "unknown")
        except OSError:
            name = "unknown"
    parts = [name]
    if "CPU family" in fields:
        parts.append(f"family {fields['CPU family']} model {fields.get('Model', '?')} "
                     f"stepping {fields.get('Stepping', '?')}")
    if "Socket(s)" in fields:
        parts.append(f"{fields['Socket(s)']} socket(s) x {fields.get('Core(s) per socket', '?')} cores x "
                     f"{fields.get('Thread(s) per core', '?')} threads")
    if "L3 cache" in fields:
        parts.append(f"L3 {fields['L3 cache']}")
    if "Hypervisor vendor" in fields:
        parts.append(f"virtual machine ({fields['Hypervisor vendor']})")
    return "; ".join(parts)


def cpu_baseline(cfg, budget_s=2.0, max_steps=2000):
    """The oracle, as it stands, on the same rank's shard (C1, C2 whole; the
    larger shards on their first CPU_SAMPLE parameters): as many full steps
    as fit in about budget_s seconds of host time (after one untimed step),
    with 1 thread and with N threads (N = OMP_NUM_THREADS if set, else the
    CPU count)."""
    import numpy as np
    import oracle
    import synth

    W = cfg.W
    begin, end = cfg.shard
    S = end - begin
    n = S if CPU_SAMPLE[cfg.name] is None else min(S, CPU_SAMPLE[cfg.name])
    grads = [synth.bf16(n, synth.grad_key(cfg.seed, 1, w), begin, cfg.sigma, cfg.outlier_pct) for w in range(W)]
    master0 = synth.f32(n, synth.master_key(cfg.seed), begin, cfg.master_sigma)
    mvd = np.uint16 if cfg.mv_bf16 else np.float32
    n_max = min(int(os.environ.get("OMP_NUM_THREADS") or 0) or (os.cpu_count() or 1), os.cpu_count() or 1)
    out = {}
    for threads in (1, n_max):
        used = oracle.threads(threads)
        master = master0.copy()
        m, v = np.zeros(n, mvd), np.zeros(n, mvd)
        param = np.zeros(n, np.uint16)
        rs = np.zeros(W)
        # one untimed step first: it takes the page faults of the new arrays
        oracle.step(grads, master, m, v, param, cfg.hparams(1), rs, cfg.rank % W)
        steps = 0
        t0 = time.perf_counter()
        while True:
            oracle.step(grads, master, m, v, param, cfg.hparams(steps + 2), rs, cfg.rank % W)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or steps >= max_steps:
                break
        out[threads] = {"value": n * steps / el, "cores": used, "steps": steps, "seconds": el}
    whole = "the whole shard" if n == S else f"the first {n:,} parameters of the shard"
    return {"value": out[n_max]["value"], "unit": "params/s", "cores": out[n_max]["cores"], "kind": "oracle",
            "sample": f"{out[n_max]['steps']} full oracle steps (reduce, norm, clip, AdamW, bf16) on {whole} "
                      f"({cfg.workload}), {out[n_max]['seconds']:.1f} s on {out[n_max]['cores']} threads",
            "single_thread": {"value": out[1]["value"], "unit": "params/s", "cores": out[1]["cores"],
                              "sample": f"{out[1]['steps']} steps on {whole}, {out[1]['seconds']:.1f} s"},
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}


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
    """Median FETCH_SIZE / WRITE_SIZE per dispatch of the step's update and
    reduce kernels, scaled by what the same counters read for a torch.neg over
    CALIB_BYTES (a plain copy: CALIB_BYTES read, CALIB_BYTES written),
    appended to out_path as update_* and reduce_* lines."""
    fetch, write = read_pmc_dir(fetch_dir), read_pmc_dir(write_dir)

    def pick(d, key):
        for k, v in d.items():
            if key in k:
                return k, v
        raise SystemExit(f"no kernel matching {key!r} in {list(d)[:10]}")

    _, cf = pick(fetch, "neg_kernel")
    _, cw = pick(write, "neg_kernel")
    f_scale = (CALIB_BYTES / 1024.0) / statistics.median(cf)
    w_scale = (CALIB_BYTES / 1024.0) / statistics.median(cw)
    lines = [f"kernel_source_hash = {kernel_source_hash()}",
             f"# calibration: torch.neg over {CALIB_BYTES} B fp32 reads FETCH_SIZE {statistics.median(cf):.1f} KiB "
             f"and WRITE_SIZE {statistics.median(cw):.1f} KiB; scale fetch x{f_scale:.4f}, write x{w_scale:.4f}"]
    for label, key in (("update", UPDATE_KERNEL), ("reduce", REDUCE_KERNEL)):
        kf, vf = pick(fetch, key)
        _, vw = pick(write, key)
        lines += [f"# {label}: {kf[:110]}",
                  f"# raw per dispatch (median of {len(vf)}): FETCH_SIZE {statistics.median(vf):.1f} KiB, "
                  f"WRITE_SIZE {statistics.median(vw):.1f} KiB",
                  f"{label}_fetch_bytes = {statistics.median(vf) * 1024 * f_scale:.0f}",
                  f"{label}_write_bytes = {statistics.median(vw) * 1024 * w_scale:.0f}"]
    with open(out_path, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_kt(kt_dir, out_path):
    """Per-kernel dispatch statistics from a rocprofv3 --kernel-trace output dir,
    split by grid size (the whole-shard reduce and the bucket reduces are the
    same kernel at different grids), appended to out_path."""
    rows = {}
    for f in glob.glob(os.path.join(kt_dir, "**", "*kernel_trace*.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                short = name.replace("void ", "").replace("z1::(anonymous namespace)::", "")
                short = short.replace("(anonymous namespace)::", "").split("(")[0]
                grid = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                rows.setdefault((short, grid), []).append(dur)
    lines = [f"{'kernel':<48} | {'workgroups':>10} | {'calls':>5} | {'avg_us':>9} | {'median_us':>9} | "
             f"{'min_us':>9} | {'max_us':>9}"]
    for (short, grid), d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{short[:48]:<48} | {grid:>10} | {len(d):>5} | {sum(d) / len(d):>9.2f} | "
                     f"{statistics.median(d):>9.2f} | {min(d):>9.2f} | {max(d):>9.2f}")
    with open(out_path, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_from_summary(path, kernel):
    """Counter bytes per launch of the step's `kernel` ("update" or "reduce")
    from the committed summary, or None if the kernels changed since the
    counters were taken."""
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
        return float(kv[f"{kernel}_fetch_bytes"]) + float(kv[f"{kernel}_write_bytes"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------- graph replay
def graph_timing(torch, z, cfg, st, design, k0, replays=40, per_graph=10):
    """The launch-bound path: per_graph consecutive steps captured once into
    one HIP graph (torch.cuda.graph), each step reading its fp32 scalars
    (t, learning rate) from its own 40-byte slot of device memory
    (zero1_hparams.device_scalars); before every replay the next per_graph
    steps' scalars are derived on the host and copied in (one stream-ordered
    copy from pinned memory, inside the timed region).  Returns ms per step."""
    W, rank = st["W"], st["rank"]
    copies = st["copies"]
    dev = copies[0].master.device
    slot = 40
    dev_scal = torch.zeros(per_graph * slot // 8, dtype=torch.float64, device=dev)
    host = torch.zeros(per_graph * slot, dtype=torch.uint8).pin_memory()
    base = dev_scal.data_ptr()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(per_graph):
            c = copies[j % len(copies)]
            z.mta_step(c.grads, c.begin, c.plan, {"device_scalars": base + slot * j}, c.rsd, W, rank,
                       flags=design, ws=c.ws)
    torch.cuda.synchronize()

    def fill(t0):
        buf = bytearray()
        for j in range(per_graph):
            buf += bytes(z.step_scalars_derive(cfg.hparams(t0 + j)))
        host.copy_(torch.frombuffer(buf, dtype=torch.uint8))
        dev_scal.view(torch.uint8).copy_(host, non_blocking=True)

    fill(k0 + 1)
    graph.replay()
    torch.cuda.synchronize()
    t = k0 + 1 + per_graph
    t_start = time.perf_counter()
    for _ in range(replays):
        fill(t)
        graph.replay()
        t += per_graph
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t_start) * 1e3 / (replays * per_graph)
    del graph
    return {"steps_per_graph": per_graph, "replays": replays, "ms_per_step": ms}


# ---------------------------------------------------------------------- bucketed flow
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
        z.mta_update(c.grads, c.begin, c.plan, cfg.hparams(k + 1), c.rsd, W, flags=z.STORE_G, ws=c.ws,
                     stream=stream)
        ev[2 * nb].record()
        torch.cuda.synchronize()
        red_ms.append(sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(nb)))
        crit_ms.append(ev[2 * nb - 1].elapsed_time(ev[2 * nb]))
    return dict(bucket_params=b, buckets=nb, reduce_ms=sum(red_ms) / steps,
                after_backward_ms=sum(crit_ms) / steps)


def bucketed_overlap(torch, z, cfg, st, k0, steps=20, bucket_bytes=25_000_000):
    """The point of the bucketed flow: the bucket reduces run while backward
    still computes.  Backward is stood in for by one bf16 GEMM per bucket (a
    layer's weight-gradient product, 8192 tokens x 768 x 3072 on the main
    stream); each bucket's reduce is issued on a second stream once its GEMM
    has finished (an event), as a ZeRO-2 engine issues it.  Per step (ms): the
    GEMMs alone, GEMMs and bucket reduces one after the other on one stream,
    and the two streams overlapped (to the end of the last reduce), each
    followed by nothing else (the partials sum and the update after backward
    are timed by bucketed_timing)."""
    W, rank, S = st["W"], st["rank"], st["S"]
    b = max(2048, bucket_bytes // (2 * W) // 2048 * 2048)
    ranges = [(lo, min(S, lo + b)) for lo in range(0, S, b)][::-1]
    nb = len(ranges)
    dev = st["copies"][0].master.device
    x = torch.randn(8192, 768, dtype=torch.bfloat16, device=dev).t().contiguous()   # 768 x 8192
    dy = torch.randn(8192, 3072, dtype=torch.bfloat16, device=dev)                   # 8192 x 3072
    dw = torch.empty(768, 3072, dtype=torch.bfloat16, device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=dev)        # default priority
    done = [torch.cuda.Event() for _ in range(nb)]

    def buckets(c, stream):
        for i, (lo, hi) in enumerate(ranges):
            yield i, lambda lo=lo, hi=hi, i=i: z.mta_reduce_range(
                [g.data_ptr() + 2 * (c.begin + lo) for g in c.grads], c.plan, lo, hi,
                c.parts.data_ptr() + 8 * (nb - 1 - i), flags=z.STORE_G, ws=c.ws, stream=stream.cuda_stream)

    def one(k, mode):
        c = st["copies"][k % len(st["copies"])]
        if not hasattr(c, "parts"):
            c.parts = torch.zeros(nb, dtype=torch.float64, device=dev)
        for i, call in buckets(c, side if mode == "overlap" else main):
            torch.mm(x, dy, out=dw)
            if mode == "gemm":
                continue
            if mode == "overlap":
                done[i].record(main)
                side.wait_event(done[i])
            call()

    out = {"bucket_params": b, "buckets": nb, "gemm": "bf16 768x8192 @ 8192x3072 per bucket"}
    for mode in ("gemm", "sequential", "overlap"):
        one(k0, mode)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(k0, k0 + steps):
            one(k, mode)
        torch.cuda.synchronize()
        out[f"{mode}_ms"] = (time.perf_counter() - t0) * 1e3 / steps
    del x, dy, dw
    return out


# ---------------------------------------------------------------------- calibrate mode
def calibrate(torch, dev, gib=4, spacing_gib=40):
    """Plain read, write and copy rates of the calibration kernel (the step
    kernels' access pattern, nothing computed) over `gib` GiB per fp32
    stream, in two layouts: packed (one torch allocation per buffer) and
    spaced (buffers spacing_gib GiB apart inside one allocation, like
    zero1_arena_plan's spaced arrays); plus two mixes shaped like the step's
    kernels: the store-g update (g, master, m, v read; master, m, v written in
    place; bf16 parameters written) and the 8-slice reduce (8 bf16 slices
    read, fp32 g written; spaced: g in the first slot, the slices packed from
    the fifth, as the arena places them).  Then the update mix at a range of
    spacings (spacing_sweep).  Returns a dict of GB/s."""
    n = (gib << 30) // 4 // 2048 * 2048          # elements per buffer
    n_tiles = n // 2048
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid, split = 8 * cus, 8
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    # name: (buffers as (bytes per element, spaced slot or None = packed after
    # the previous buffer), reads as (buffer, bytes), writes likewise)
    shapes = {
        "read": ([(4, 0)], [(0, 4)], []),
        "write": ([(4, 0)], [], [(0, 4)]),
        "copy": ([(4, 0), (4, 1)], [(0, 4)], [(1, 4)]),
        "update_mix": ([(4, 0), (4, 1), (4, 2), (4, 3), (2, 4)],
                       [(0, 4), (1, 4), (2, 4), (3, 4)], [(1, 4), (2, 4), (3, 4), (4, 2)]),
        "reduce8_mix": ([(4, 0)] + [(2, 4)] + [(2, None)] * 7,
                        [(k, 2) for k in range(1, 9)], [(0, 4)]),
    }
    out = {"elements_per_buffer": n, "workgroups": grid}
    unit = 2 << 20
    for layout in ("packed", "spaced"):
        for name, (bufspec, rspec, wspec) in shapes.items():
            sizes = [n * b for b, _ in bufspec]
            if layout == "packed":
                bufs = [torch.empty(sz, dtype=torch.uint8, device=dev) for sz in sizes]
                addrs = [t.data_ptr() for t in bufs]
            else:
                offs, pos = [], 0
                for sz, (_, slot) in zip(sizes, bufspec):
                    o = slot * (spacing_gib << 30) if slot is not None else (pos + unit - 1) // unit * unit
                    offs.append(o)
                    pos = o + sz
                arena = torch.empty(max(o + sz for o, sz in zip(offs, sizes)), dtype=torch.uint8, device=dev)
                addrs = [arena.data_ptr() + o for o in offs]
                bufs = [arena]
            for buf in bufs:
                buf.fill_(0x3c)
            del buf
            rd = [(addrs[i], b, False) for i, b in rspec]
            wr = [(addrs[i], b, False) for i, b in wspec]
            ms, U = best_calibration(torch, rd, wr, n_tiles, grid, split, sink.data_ptr(), stream, reps=5)
            nbytes = n_tiles * 2048 * (sum(b for _, b in rspec) + sum(b for _, b in wspec))
            out[f"{layout}_{name}_GBps"] = nbytes / (ms * 1e-3) / 1e9
            out[f"{layout}_{name}_tiles_in_flight"] = U
            log(f"calibrate {layout} {name}: {out[f'{layout}_{name}_GBps']:.0f} GB/s (U={U})")
            del bufs, addrs, rd, wr
            arena = None
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    out["update_mix_by_spacing_GBps"] = spacing_sweep(torch, dev, sink, stream, cus)
    out["update_mix_by_cache_policy_GBps"] = policy_sweep(torch, dev, stream, cus)
    out["update_mix_random_placements"] = placement_search(torch, dev, stream, cus)
    return out


def placement_search(torch, dev, stream, cus, n_placements=40, seed=7, span_gib=200, min_gap_gib=5):
    """The W=1 update mix (zcal_policy_mix, nt loads and stores) over 1 GiB
    fp32 streams placed at random whole-GiB offsets inside one span_gib GiB
    allocation (each stream at least min_gap_gib GiB from the next), against
    the planner's uniform 40 GiB spacing: {"uniform_40_GBps", "placements":
    [[offsets in GiB of g, p, m, v, out], GB/s] ...}."""
    import numpy as np
    GiB = 1 << 30
    n = GiB // 4 // 2048 * 2048
    n_tiles = n // 2048
    arena = torch.empty(span_gib * GiB, dtype=torch.uint8, device=dev)
    arena.fill_(0x3c)
    base = (arena.data_ptr() + (2 << 20) - 1) // (2 << 20) * (2 << 20)
    assert base - arena.data_ptr() + (span_gib - 2) * GiB + 4 * n <= span_gib * GiB

    def rate(offs):
        ptr = [base + o * GiB for o in offs]
        fn = lambda: zcal_policy_mix(2, 2, *ptr, n_tiles, 8 * cus, 8, stream)  # noqa: E731
        fn()
        torch.cuda.synchronize()
        return n_tiles * 2048 * 28 / (timed_passes(torch, fn, 5) * 1e-3) / 1e9

    rng = np.random.default_rng(seed)
    res = {"uniform_40_GBps": rate([0, 40, 80, 120, 160]), "placements": []}
    for _ in range(n_placements):
        while True:
            offs = sorted(int(x) for x in rng.choice(span_gib - 2, size=5, replace=False))
            if all(b - a >= min_gap_gib for a, b in zip(offs, offs[1:])):
                break
        o = [offs[i] for i in rng.permutation(5)]
        res["placements"].append([o, rate(o)])
    rates = sorted(r for _, r in res["placements"])
    log(f"calibrate update mix, {n_placements} random placements: min {rates[0]:.0f}, median "
        f"{rates[len(rates) // 2]:.0f}, max {rates[-1]:.0f} GB/s; uniform 40 GiB {res['uniform_40_GBps']:.0f}")
    del arena
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


POLICY_NAMES = {0: "none", 1: "sc0", 2: "nt", 3: "sc0 nt", 16: "sc1", 17: "sc0 sc1", 18: "nt sc1",
                19: "sc0 nt sc1"}


def policy_sweep(torch, dev, stream, cus, spacing_gib=40):
    """The recompute design's update mix at W = 1 (a bf16 gradient read;
    master, m, v read and rewritten; bf16 parameters written: 28 bytes per
    element) over 1 GiB fp32 streams spacing_gib GiB apart, for each pair of
    cache policies on its loads and its stores: {"load / store": GB/s}."""
    n = (1 << 30) // 4 // 2048 * 2048
    n_tiles = n // 2048
    D = spacing_gib << 30
    arena = torch.empty(4 * D + 2 * n, dtype=torch.uint8, device=dev)
    arena.fill_(0x3c)
    g, p, m, v, o = (arena.data_ptr() + k * D for k in range(5))
    res = {}
    for rp in (2, 0, 16, 18):
        for wp in (2, 0, 1, 16, 17, 18):
            fn = lambda: zcal_policy_mix(rp, wp, g, p, m, v, o, n_tiles, 8 * cus, 8, stream)  # noqa: E731
            fn()
            torch.cuda.synchronize()
            ms = timed_passes(torch, fn, 5)
            key = f"{POLICY_NAMES[rp]} / {POLICY_NAMES[wp]}"
            res[key] = n_tiles * 2048 * 28 / (ms * 1e-3) / 1e9
            log(f"calibrate update mix, loads {POLICY_NAMES[rp]}, stores {POLICY_NAMES[wp]}: {res[key]:.0f} GB/s")
    del arena
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def spacing_sweep(torch, dev, sink, stream, cus, spacings_gib=(1, 2, 4, 8, 12, 16, 20, 24, 32, 40, 48)):
    """The update mix (g, master, m, v read; master, m, v rewritten; bf16
    written) over 1 GiB fp32 streams placed D GiB apart in one allocation, for
    each D: {D: GB/s}."""
    n = (1 << 30) // 4 // 2048 * 2048
    n_tiles = n // 2048
    dmax = max(spacings_gib) << 30
    arena = torch.empty(4 * dmax + 2 * n, dtype=torch.uint8, device=dev)
    arena.fill_(0x3c)
    base = arena.data_ptr()
    res = {}
    for D in spacings_gib:
        o = [k * (D << 30) for k in range(5)]
        rd = [(base + o[k], 4, False) for k in range(4)]
        wr = [(base + o[k], 4, False) for k in (1, 2, 3)] + [(base + o[4], 2, False)]
        ms, _ = best_calibration(torch, rd, wr, n_tiles, 8 * cus, 8, sink.data_ptr(), stream, reps=5)
        res[D] = n_tiles * 2048 * 30 / (ms * 1e-3) / 1e9
        log(f"calibrate update mix, streams {D} GiB apart: {res[D]:.0f} GB/s")
    del arena
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--layout", choices=["arena", "packed", "both"], default="both",
                    help="arena: arrays placed by zero1_arena_plan; packed: one torch allocation each")
    ap.add_argument("--no-per-config", action="store_true", help="the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--summarize-kt", nargs=2, metavar=("KT_DIR", "OUT"))
    a = ap.parse_args()

    if a.summarize_pmc:
        summarize_pmc(*a.summarize_pmc)
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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.calibrate:
        out = {"calibrate": calibrate(torch, dev), "device": torch.cuda.get_device_properties(dev).name}
        print(json.dumps(out), flush=True)
        return 0

    cfgs = configs()
    cfg = cfgs[a.config]
    if a.pmc_run:
        st = setup(torch, cfg, z.STORE_G if cfg.W > 4 else z.RECOMPUTE_G, 1, dev,
                   "packed" if a.layout == "packed" else "arena")
        run_steps(z, cfg, st, z.STORE_G if cfg.W > 4 else z.RECOMPUTE_G, 0, 4)
        x = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print("pmc run done", flush=True)
        return 0

    layouts = ["arena", "packed"] if a.layout == "both" else [a.layout]

    def steps_for(name):
        return max(a.steps, MIN_STEPS.get(name, 0))

    # the headline workload: exactly --steps timed steps after --warmup, per layout
    head = {}
    for lay in layouts:
        log(f"{cfg.name} {lay}: setup + {a.warmup} warmup + {a.steps} timed steps")
        head[lay] = measure(torch, z, cfg, lay, a.steps, a.warmup, dev, bucketed=(cfg.name == "C2"))
        log(f"{cfg.name} {lay}: {head[lay]['ms_per_step']:.4f} ms/step, "
            f"{head[lay]['pct_of_peak_hbm']:.1f}% of 8 TB/s")
    main_lay = layouts[0]
    h = head[main_lay]
    S, W = cfg.S, cfg.W
    upd = h["kernels"]["update"]
    out = {
        "metric": "params updated/s and achieved HBM GB/s (% of peak) per fused ZeRO-1 step",
        "value": h["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64 Irwin-Hall gradients and masters; tensor shapes only, no weights)",
        "config": {
            "workload": cfg.workload, "W": W, "rank": cfg.rank, "shard_params": S,
            "bytes_per_param": cfg.bytes_per_param, "design": "store_g" if W > 4 else "recompute_g",
            "m_v": "bf16" if cfg.mv_bf16 else "fp32", "memory_layout": h["layout"],
        },
        "algorithmic_GBps": h["algorithmic_GBps"],
        "pct_of_peak_hbm": h["pct_of_peak_hbm"],
        "gpu_ms_per_step": h["gpu_ms_per_step"],
        "roofline": {"bound": "hbm", "kernel": UPDATE_KERNEL, "achieved": upd["algorithmic_GBps"],
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": upd["algorithmic_GBps"] / PEAK_HBM_GBS,
                     "traffic": upd["traffic"], "algorithmic_bytes_per_launch": upd["algorithmic_bytes"],
                     "kernel_ms": upd["ms"], "calibrated_ms": upd.get("calibrated_ms"),
                     "calibrated_over_kernel": upd.get("calibrated_over_kernel")},
        "kernels": h["kernels"],
        "calibrated_ms_per_step": h.get("calibrated_ms_per_step"),
        "layouts": {lay: {k: head[lay][k]
                          for k in ("ms_per_step", "params_per_s", "pct_of_peak_hbm", "layout", "other_tensors",
                                    "mall_warm_ms_per_step") if k in head[lay]}
                    for lay in layouts},
    }
    for extra in ("bucketed", "graph"):
        if extra in h:
            out[extra] = h[extra]
    if not a.no_per_config:
        per = {}
        for name in PER_CONFIG:
            if name == cfg.name:
                continue
            c = cfgs[name]
            per[name] = {"workload": c.workload, "W": c.W, "shard_params": c.S, "bytes_per_param": c.bytes_per_param,
                         "design": "store_g" if c.W > 4 else "recompute_g"}
            for lay in layouts:
                k = steps_for(name)
                log(f"{name} {lay}: setup + {a.warmup} warmup + {k} timed steps")
                r = measure(torch, z, c, lay, k, a.warmup, dev, bucketed=(name == "C2"))
                log(f"{name} {lay}: {r['ms_per_step']:.4f} ms/step, {r['pct_of_peak_hbm']:.1f}% of 8 TB/s")
                per[name][lay] = r
        out["per_config"] = per
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle, 1 thread and N threads)")
        out["cpu_baseline"] = cpu_baseline(cfg)
        if not a.no_per_config:
            for name in PER_CONFIG:
                if name in out.get("per_config", {}):
                    out["per_config"][name]["cpu_baseline"] = cpu_baseline(cfgs[name])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
