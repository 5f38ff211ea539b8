"""Drive the oracle over all W simulated ranks of a small flat workload.

Test infrastructure: builds each step's W replica gradients with ``synth`` (or a
caller-supplied function), forms every rank's partial sum of squares with the
oracle, then runs each requested rank's step with the oracle.  The result is the
per-rank state after ``steps`` steps plus the per-step norm information.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from synth.workloads import shard_range


class RankState:
    def __init__(self, master, mv_bf16=False):
        n = master.size
        self.master = master.astype(np.float32).copy()
        if mv_bf16:
            self.m = np.zeros(n, dtype=np.uint16)
            self.v = np.zeros(n, dtype=np.uint16)
        else:
            self.m = np.zeros(n, dtype=np.float32)
            self.v = np.zeros(n, dtype=np.float32)
        self.param = oracle.f32_to_bf16(self.master)
        self.infos = []


def synth_grads(seed, t, W, N, sigma, outlier_pct=0):
    return [synth.bf16(N, synth.grad_key(seed, t, w), 0, sigma, outlier_pct) for w in range(W)]


def run(N, W, steps, grads_fn, master_full, hp_fn, ranks=None, mv_bf16=False, average=True):
    """grads_fn(t) -> list of W uint16 arrays of length N (full replica gradients)."""
    ranks = list(range(W)) if ranks is None else list(ranks)
    states = {}
    for r in ranks:
        b, e = shard_range(N, W, r)
        states[r] = RankState(master_full[b:e], mv_bf16)
    for t in range(1, steps + 1):
        G = grads_fn(t)
        partials = np.zeros(W, dtype=np.float64)
        for r in range(W):
            b, e = shard_range(N, W, r)
            if e > b:
                partials[r] = oracle.sumsq(oracle.shard_reduce([g[b:e] for g in G], average))
        for r in ranks:
            b, e = shard_range(N, W, r)
            st = states[r]
            if e == b:
                continue
            rs = partials.copy()
            info = oracle.step([g[b:e] for g in G], st.master, st.m, st.v, st.param,
                               hp_fn(t), rs, r, average=average)
            assert rs[r] == partials[r]
            st.infos.append(info)
    return states
