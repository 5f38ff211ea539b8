"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times (zero1_mta_step over the rank's piece list, the library's default
design), against the CPU oracle.

* GPT-2 small, W=8 (124,439,808 params): rank 4 for 10 steps and every rank
  for 2 steps, full shards compared element by element.
* 7.5e9 params, W=64, rank 0 (117,187,500-param shard; 64 slices = 15 GB);
  Llama-7B, W=8, rank 3 (842,301,952 params, 40 pieces) and rank 0;
  7e9 params, W=1, with fp32 and with bf16 m, v (112 GB / 84 GB of state).
  Each step's exact norm comes from the oracle streaming the whole shard
  (reduce + fp64 sum of squares, on host copies of the seeded gradients, which
  are spot-checked against the CPU generator); the exact state trajectory is
  tracked by the oracle on a sampled subset (the first and last 2^20
  elements, every 997th element, and 4096 elements on each side of every
  piece boundary) whose gradients are drawn on the CPU.  GPU state on the
  subset must match bit for bit; norms to 1e-12 relative, clip decision and
  coefficient exactly.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import oracle
import synth
import zero_sharded_mixed_zero1_amd as z
from synth.workloads import configs, shard_range
from tests.gpu_util import assert_bf16_equal, assert_f32_equal, rel_close, torch_cuda, ws_tensor

pytestmark = [pytest.mark.gpu, pytest.mark.large]

NORM_TOL = 1e-12
CHUNK = 1 << 22          # host streaming chunk (a multiple of the oracle's 65,536-element norm block)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return torch, dev


class Shard:
    """One rank's shard of a config on the GPU: W gradient slices (or all
    replicas' full buffers), flat master/m/v, the bf16 parameters of the
    tensors the shard touches, and the multi-tensor plan."""

    def __init__(self, torch, dev, cfg, rank, full_replicas=False):
        self.torch, self.dev, self.cfg, self.rank = torch, dev, cfg, rank
        numels = [n for _, n in cfg.tensors]
        self.N = sum(numels)
        self.begin, self.S = z.shard_range(self.N, cfg.W, rank)
        self.pl = z.shard_pieces(numels, self.begin, self.begin + self.S)
        offs = np.concatenate([[0], np.cumsum(numels)])
        self.piece_starts = [so for ti, off, so, n in self.pl]
        first, last = self.pl[0][0], self.pl[-1][0]
        self.p_lo = int(offs[first])
        self.params = torch.zeros(int(offs[last + 1]) - self.p_lo, dtype=torch.int16, device=dev)
        self.master = torch.empty(self.S, dtype=torch.float32, device=dev)
        synth.fill_f32_(self.master, synth.master_key(cfg.seed), self.begin, cfg.master_sigma)
        mvdt = torch.int16 if cfg.mv_bf16 else torch.float32
        self.m = torch.zeros(self.S, dtype=mvdt, device=dev)
        self.v = torch.zeros(self.S, dtype=mvdt, device=dev)
        pieces = [(n, so, self.params[self.begin + so - self.p_lo:], self.master[so:], self.m[so:], self.v[so:])
                  for ti, off, so, n in self.pl]
        self.table = ws_tensor(torch, z.mta_table_bytes(pieces), dev)
        self.plan = z.mta_plan(pieces, self.table, flags=z.MV_BF16 if cfg.mv_bf16 else 0)
        self.ws = ws_tensor(torch, z.mta_workspace_bytes(self.plan, cfg.W), dev)
        self.full_replicas = full_replicas
        if full_replicas:
            self.grads = [torch.empty(self.N, dtype=torch.int16, device=dev) for _ in range(cfg.W)]
            self.gbegin = self.begin
        else:
            self.grads = [torch.empty(self.S, dtype=torch.int16, device=dev) for _ in range(cfg.W)]
            self.gbegin = 0

    def fill_grads(self, t):
        c = self.cfg
        for w, g in enumerate(self.grads):
            i0 = 0 if self.full_replicas else self.begin
            synth.fill_bf16_(g, synth.grad_key(c.seed, t, w), i0, c.sigma, c.outlier_pct)

    def slice_host(self, w, lo, hi):
        """Host copy of replica w's gradient at shard positions [lo, hi)."""
        off = self.gbegin
        return self.grads[w][off + lo:off + hi].cpu().numpy().view(np.uint16)

    def step(self, t, rank_sumsq, info):
        z.mta_step(self.grads, self.gbegin, self.plan, self.cfg.hparams(t), rank_sumsq, self.cfg.W, self.rank,
                   info_out=info, ws=self.ws)

    def state_at(self, idx):
        t = self.torch
        ii = t.from_numpy(idx).to(self.dev)
        master = self.master.index_select(0, ii).cpu().numpy()
        m = self.m.index_select(0, ii).cpu().numpy()
        v = self.v.index_select(0, ii).cpu().numpy()
        p = self.params.index_select(0, ii + (self.begin - self.p_lo)).cpu().numpy().view(np.uint16)
        if self.cfg.mv_bf16:
            m, v = m.view(np.uint16), v.view(np.uint16)
        return master, m, v, p


def streamed_partial(sh: Shard, rng, t: int) -> float:
    """Oracle: this rank's fp64 sum of squares over the whole shard, streamed
    through the host in norm-block-aligned chunks; spot-checks the copied
    gradients against the CPU generator."""
    c = sh.cfg
    total = 0.0
    for lo in range(0, sh.S, CHUNK):
        hi = min(lo + CHUNK, sh.S)
        G = [sh.slice_host(w, lo, hi) for w in range(c.W)]
        for w in rng.choice(c.W, size=min(c.W, 4), replace=False):
            k = rng.integers(0, hi - lo, size=64)
            exp = synth.bf16_at(sh.begin + lo + k, synth.grad_key(c.seed, t, int(w)), c.sigma, c.outlier_pct)
            assert np.array_equal(G[w][k], exp), "GPU-drawn gradients differ from the CPU generator"
        total = oracle.sumsq(oracle.shard_reduce(G), total)
    return total


def subset_indices(sh: Shard, every=997, edge=1 << 20, around=4096):
    S = sh.S
    parts = [np.arange(0, min(edge, S)), np.arange(max(0, S - edge), S), np.arange(0, S, every)]
    for ps in sh.piece_starts[1:]:
        parts.append(np.arange(max(0, ps - around), min(S, ps + around)))
    return np.unique(np.concatenate(parts)).astype(np.int64)


def run_large(env, cfg, rank, steps, norms_cache=None):
    torch, dev = env
    t0 = time.time()
    sh = Shard(torch, dev, cfg, rank)
    idx = subset_indices(sh)
    gidx = sh.begin + idx
    o_master = synth.f32_at(gidx, synth.master_key(cfg.seed), cfg.master_sigma)
    mvd = np.uint16 if cfg.mv_bf16 else np.float32
    o_m, o_v = np.zeros(idx.size, mvd), np.zeros(idx.size, mvd)
    o_p = np.zeros(idx.size, np.uint16)
    rsd = torch.zeros(cfg.W, dtype=torch.float64, device=dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    rng = np.random.default_rng(cfg.seed + rank)
    log(f"[{cfg.name} rank {rank}] shard {sh.S:,} params, {len(sh.pl)} pieces, subset {idx.size:,}, "
        f"setup {time.time() - t0:.1f}s")
    for t in range(1, steps + 1):
        ts = time.time()
        sh.fill_grads(t)
        torch.cuda.synchronize()
        key = (cfg.seed, rank, t)
        if norms_cache is not None and key in norms_cache:
            q = norms_cache[key]
        else:
            q = streamed_partial(sh, rng, t)
            if norms_cache is not None:
                norms_cache[key] = q
        rs = np.zeros(cfg.W)
        rs[rank] = q                                   # other ranks' partials: 0 (shard-local norm)
        norm = oracle.global_norm(rs)
        clip, coef = oracle.clip_coef(norm, cfg.max_norm)
        # GPU step (its rank_sumsq entry is overwritten with its own partial)
        rsd.zero_()
        sh.step(t, rsd, info)
        torch.cuda.synchronize()
        ni = info.cpu().numpy()
        assert rel_close(ni[1], norm, NORM_TOL), (t, ni[1], norm)
        assert rel_close(rsd[rank].item(), q, NORM_TOL)
        assert bool(ni[2:4].view(np.int32)[1]) == clip
        assert ni[2:3].view(np.float32)[0] == coef
        # oracle trajectory on the subset
        G = [synth.bf16_at(gidx, synth.grad_key(cfg.seed, t, w), cfg.sigma, cfg.outlier_pct) for w in range(cfg.W)]
        g = oracle.shard_reduce(G)
        s = oracle.adamw_scalars(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, t)
        oracle.adamw(g, o_master, o_m, o_v, o_p, s, clip, coef)
        log(f"[{cfg.name} rank {rank}] step {t}: norm {norm:.6g} clip {clip} coef {float(coef):.6g} "
            f"({time.time() - ts:.1f}s)")
    master, m, v, p = sh.state_at(idx)
    what = f"{cfg.name} rank {rank} after {steps} steps"
    assert_f32_equal(master, o_master, "master " + what)
    if cfg.mv_bf16:
        assert_bf16_equal(m, o_m, "m " + what)
        assert_bf16_equal(v, o_v, "v " + what)
    else:
        assert_f32_equal(m, o_m, "m " + what)
        assert_f32_equal(v, o_v, "v " + what)
    assert_bf16_equal(p, o_p, "param " + what)
    del sh
    torch.cuda.empty_cache()
    log(f"[{cfg.name} rank {rank}] ok in {time.time() - t0:.1f}s")


# ---------------------------------------------------------------- GPT-2 small, full shards
def test_gpt2_small_w8_full_shards(env):
    torch, dev = env
    cfg = configs()["C2"]
    W, N = cfg.W, cfg.n_total
    from tests.oracle_sim import RankState
    ranks_all_steps = {4: cfg.steps}
    for r in range(W):
        ranks_all_steps.setdefault(r, 2)
    shards = {r: Shard(torch, dev, cfg, r, full_replicas=(r == 0)) for r in range(W)}
    full = shards[0].grads                          # every replica's full gradient (one copy on the GPU)
    for r in range(1, W):
        shards[r].grads = full
        shards[r].gbegin = shards[r].begin
    ost = {r: RankState(synth.f32(shards[r].S, synth.master_key(cfg.seed), shards[r].begin, cfg.master_sigma))
           for r in range(W)}
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    ws_r = ws_tensor(torch, z.workspace_bytes(shards[0].S + 8, W), dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    for t in range(1, cfg.steps + 1):
        ts = time.time()
        G = [synth.bf16(N, synth.grad_key(cfg.seed, t, w), 0, cfg.sigma, cfg.outlier_pct) for w in range(W)]
        for w, g in enumerate(full):
            synth.fill_bf16_(g, synth.grad_key(cfg.seed, t, w), 0, cfg.sigma, cfg.outlier_pct)
        part = np.zeros(W)
        for r in range(W):
            b, e = shard_range(N, W, r)
            part[r] = oracle.sumsq(oracle.shard_reduce([g[b:e] for g in G]))
            z.shard_reduce(full, b, e - b, sumsq_out=rsd[r:r + 1], ws=ws_r)
        torch.cuda.synchronize()
        gpu_part = rsd.cpu().numpy().copy()
        for r in range(W):
            assert rel_close(gpu_part[r], part[r], NORM_TOL)
        hp = cfg.hparams(t)
        for r in range(W):
            if t > ranks_all_steps[r]:
                continue
            b, e = shard_range(N, W, r)
            rs = part.copy()
            oi = oracle.step([g[b:e] for g in G], ost[r].master, ost[r].m, ost[r].v, ost[r].param, hp, rs, r)
            rsd.copy_(torch.from_numpy(gpu_part))
            shards[r].step(t, rsd, info)
            torch.cuda.synchronize()
            ni = info.cpu().numpy()
            assert rel_close(ni[1], oi.norm, NORM_TOL)
            assert bool(ni[2:4].view(np.int32)[1]) == oi.clip and oi.clip
            assert ni[2:3].view(np.float32)[0] == oi.coef
        log(f"[GPT-2 small W=8] step {t}: norm {oi.norm:.6g} coef {float(oi.coef):.6g} ({time.time() - ts:.1f}s)")
    for r in range(W):
        sh = shards[r]
        idx = np.arange(sh.S, dtype=np.int64)
        master = sh.master.cpu().numpy()
        m = sh.m.cpu().numpy()
        v = sh.v.cpu().numpy()
        p = sh.params[sh.begin - sh.p_lo:sh.begin - sh.p_lo + sh.S].cpu().numpy().view(np.uint16)
        what = f"C2 rank {r} after {ranks_all_steps[r]} steps"
        assert_f32_equal(master, ost[r].master, "master " + what)
        assert_f32_equal(m, ost[r].m, "m " + what)
        assert_f32_equal(v, ost[r].v, "v " + what)
        assert_bf16_equal(p, ost[r].param, "param " + what)
        del idx


# ---------------------------------------------------------------- the multi-GB shards
def test_dense_7p5b_w64_rank0(env):
    c = configs()["C3"]
    run_large(env, c, 0, c.steps)


def test_dense_7p5b_w64_last_rank(env):
    c = configs()["C3"]
    run_large(env, c, 63, 2)


@pytest.mark.parametrize("rank,steps", [(3, 5), (0, 2), (7, 2)])
def test_llama7b_w8(env, rank, steps):
    c = configs()["C4"]
    run_large(env, c, rank, steps)


def test_dense_7b_w1_fp32_and_bf16_moments(env):
    cache = {}
    for name in ("C5a", "C5b"):
        c = configs()[name]
        run_large(env, c, 0, c.steps, norms_cache=cache)
