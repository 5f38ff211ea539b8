"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed operand, a contracted multiply-add, a flushed
subnormal, the wrong rounding) fails at least one of them:

(a) the four-rank collective example (reduce-scatter + all-gather = all-reduce),
(b) the bf16 stagnation example and the fp32 master that escapes it,
(c) closed-form AdamW bias correction under a constant gradient,
(d) brute force: the oracle re-evaluated in exact rational arithmetic on
    16-element shards for W in {1,2,3,4,5,8,64}, every rank, 10 steps,
plus invariants (norm scaling, post-clip norm, W=1 identity, ZeRO-1 = DDP,
update/decay order, memory accounting) and RNE against torch's bfloat16.
"""
from __future__ import annotations

import math
import os
import struct

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import shard_range
from tests import softfloat as sf
from tests.oracle_sim import run as oracle_run, synth_grads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = float(v)
    return out


def _bf16_of(values):
    """Exact bf16 bit patterns of small integers / exactly representable values."""
    x = np.asarray(values, dtype=np.float32)
    h = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(h), x), "value not exact in bf16"
    return h


HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0)


def hp_at(t, **over):
    d = dict(HP)
    d.update(over)
    d["step"] = t
    return d


# ------------------------------------------------------------------ (a)
def test_four_rank_worked_example():
    rows = []
    for line in open(os.path.join(GOLDEN, "four_rank_collectives.txt")):
        if line.startswith("#") or not line.strip():
            continue
        r, x, ar, rs, ag = (c.strip() for c in line.split("|"))
        rows.append((int(r), [float(v) for v in x.split(",")], [float(v) for v in ar.split(",")],
                     float(rs), [float(v) for v in ag.split(",")]))
    W = len(rows)
    N = W
    replicas = [_bf16_of(x) for _, x, _, _, _ in rows]
    # every rank: sum over replicas of its own block (reduce-scatter, no averaging)
    parts = []
    for r, _, _, rs_expect, _ in rows:
        b, e = shard_range(N, W, r)
        assert (b, e) == (r, r + 1)          # rank i owns block i
        got = oracle.shard_reduce([g[b:e] for g in replicas], average=False)
        assert got.tolist() == [rs_expect]
        # the average times W is the same sum, exactly
        avg = oracle.shard_reduce([g[b:e] for g in replicas], average=True)
        assert (avg * np.float32(W)).tolist() == [rs_expect]
        parts.append(got)
    gathered = np.concatenate(parts)                              # all-gather
    for _, _, ar_expect, _, ag_expect in rows:
        assert gathered.tolist() == ag_expect == ar_expect        # = all-reduce
    # non-sharded reduce of the whole vector (all-reduce) gives the same numbers
    full = oracle.shard_reduce(replicas, average=False)
    assert full.tolist() == rows[0][2]


# ------------------------------------------------------------------ (b)
def test_bf16_stagnation_example():
    g = _kv("bf16_stagnation.txt")
    steps = int(g["steps"])
    inc_bf16 = oracle.f32_to_bf16(np.array([g["increment"]], dtype=np.float32))[0]
    assert oracle.bf16_to_f32(np.array([inc_bf16]))[0] == np.float32(-0.00099945068359375)
    w = oracle.f32_to_bf16(np.array([1.0], dtype=np.float32))
    for _ in range(steps):
        s = oracle.bf16_to_f32(w) + oracle.bf16_to_f32(np.array([inc_bf16]))   # fp32 add
        w = oracle.f32_to_bf16(s.astype(np.float32))                              # back to bf16
    assert float(oracle.bf16_to_f32(w)[0]) == g["bf16_weight_after"]
    master = np.float32(1.0)
    for _ in range(steps):
        master = np.float32(master - np.float32(g["increment"] * -1.0))
    assert round(float(master), 4) == g["fp32_master_after_rounded_4dp"]
    assert abs(float(master) - 9.3246e-6) < 1e-9
    one = oracle.f32_to_bf16(np.array([1.0], dtype=np.float32))
    nxt = oracle.bf16_to_f32(one + np.uint16(1))[0]
    assert float(nxt) - 1.0 == g["bf16_eps"] == 2.0 ** -7


def test_stagnation_escaped_by_fp32_master():
    """The step lands on the fp32 master: with a constant +1e-3 gradient, lr=1e-3,
    no decay and no clip, 1000 steps walk the master from 1.0 to ~0 and the bf16
    copy follows it down instead of sticking at 1.0."""
    g = _bf16_of([2.0 ** -10])            # positive, exactly representable gradient
    master = np.array([1.0], dtype=np.float32)
    m = np.zeros(1, np.float32)
    v = np.zeros(1, np.float32)
    p = oracle.f32_to_bf16(master)
    exact = 1.0
    for t in range(1, 1001):
        hp = hp_at(t, weight_decay=0.0, max_norm=math.inf)
        rs = np.zeros(1)
        oracle.step([g], master, m, v, p, hp, rs, 0)
        # closed form of the update under a constant gradient (see test (c))
        gg = 2.0 ** -10
        bc2 = 1 - 0.95 ** t
        exact -= 1e-3 * gg * math.sqrt(bc2) / (math.sqrt(bc2) * gg + 1e-8)
    assert abs(float(master[0]) - exact) < 1e-4
    assert abs(float(master[0])) < 2e-3
    assert oracle.bf16_to_f32(p)[0] == oracle.bf16_to_f32(oracle.f32_to_bf16(master))[0]
    assert abs(float(oracle.bf16_to_f32(p)[0])) < 2e-3


# ------------------------------------------------------------------ (c)
@pytest.mark.parametrize("gval", [2.0 ** -7, -3.0 * 2.0 ** -12, 0.5])
def test_closed_form_bias_correction(gval):
    """Constant gradient g: m_t = (1-b1^t) g, v_t = (1-b2^t) g^2 exactly in real
    arithmetic, so the update is lr*g*sqrt(1-b2^t)/(sqrt(1-b2^t)|g|+eps) for
    every t; the oracle (fp32) must track an fp64 evaluation of that closed form."""
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.95, 1e-8, 0.1
    n = 1
    g = _bf16_of([gval])
    master = np.array([0.25], np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = oracle.f32_to_bf16(master)
    p64 = 0.25
    for t in range(1, 11):
        oracle.step([g], master, m, v, p, hp_at(t, max_norm=math.inf), np.zeros(1), 0)
        bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
        m64, v64 = bc1 * gval, bc2 * gval * gval
        u64 = lr * math.sqrt(bc2) / bc1 * m64 / (math.sqrt(v64) + eps)
        assert abs(u64 - lr * gval * math.sqrt(bc2) / (math.sqrt(bc2) * abs(gval) + eps)) < 1e-15
        p64 = (p64 - u64) * (1 - lr * wd)
        assert abs(float(m[0]) - m64) <= 1e-6 * abs(m64)
        assert abs(float(v[0]) - v64) <= 1e-6 * abs(v64)
        assert abs(float(master[0]) - p64) <= 1e-6 * abs(p64)
    # step 1 alone, no decay: |delta| = lr*sqrt(1-b2)|g|/(sqrt(1-b2)|g|+eps), independent of b1
    for b1x in (0.0, 0.5, 0.9, 0.99):
        mm = np.array([1.0], np.float32)
        m = np.zeros(1, np.float32)
        v = np.zeros(1, np.float32)
        oracle.step([g], mm, m, v, oracle.f32_to_bf16(mm),
                    hp_at(1, beta1=b1x, weight_decay=0.0, max_norm=math.inf), np.zeros(1), 0)
        d = lr * math.sqrt(1 - b2) * abs(gval) / (math.sqrt(1 - b2) * abs(gval) + eps)
        assert abs((1.0 - float(mm[0])) * math.copysign(1, gval) - d) <= 1e-7


def test_update_then_decay_order():
    """The page orders the decay after the update; torch decays first.  The two
    differ by sigma*q*lr*lambda per step (order lr^2*lambda)."""
    rng = np.random.default_rng(5)
    n = 4096
    g = rng.standard_normal(n).astype(np.float32) * np.float32(1e-2)
    p0 = rng.standard_normal(n).astype(np.float32)
    s = oracle.adamw_scalars(1e-3, 0.9, 0.95, 1e-8, 0.1, 3)
    pa, ma, va = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.adamw(g, pa, ma, va, np.zeros(n, np.uint16), s, False, 1.0)
    pb, mb, vb = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.adamw_decay_first(g, pb, mb, vb, s)
    assert np.array_equal(ma, mb) and np.array_equal(va, vb)
    q = ma.astype(np.float64) / (np.sqrt(va.astype(np.float64)) + 1e-8)
    expect = np.float64(s.sigma) * q * (1 - np.float64(s.delta))
    diff = pa.astype(np.float64) - pb.astype(np.float64)
    tol = 4 * np.spacing(np.abs(p0)).astype(np.float64)
    assert np.all(np.abs(diff - expect) <= tol)
    assert np.any(diff != 0)


def test_bf16_moments_are_the_fp32_step_rounded():
    """Reading 9 (bf16 m, v): each step widens the stored moments, runs the
    fp32 step, stores the nearest-even bf16 of the new moments and updates the
    master with the unrounded fp32 ones.  Checked against the fp32-moment path
    started from the same widened moments, with torch's bfloat16 conversion
    (a library routine) as the rounding reference."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    n = 20000
    master = rng.standard_normal(n).astype(np.float32) * np.float32(0.02)
    mb, vb = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    pb = np.zeros(n, np.uint16)
    for t in (1, 2, 3):
        g = (rng.standard_normal(n) * 0.05).astype(np.float32)
        s = oracle.adamw_scalars(1e-3, 0.9, 0.95, 1e-8, 0.1, t)
        pa, ma, va = master.copy(), oracle.bf16_to_f32(mb).copy(), oracle.bf16_to_f32(vb).copy()
        param_a = np.zeros(n, np.uint16)
        oracle.adamw(g, pa, ma, va, param_a, s, False, 1.0)
        oracle.adamw(g, master, mb, vb, pb, s, False, 1.0)
        rne = lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(mb, rne(ma)) and np.array_equal(vb, rne(va)), f"t={t}"
        assert np.array_equal(master.view(np.uint32), pa.view(np.uint32)), f"t={t}"
        assert np.array_equal(pb, param_a) and np.array_equal(pb, rne(master)), f"t={t}"
        assert np.any(oracle.bf16_to_f32(mb) != ma)   # the rounding is visible


def test_scalars():
    for t in (1, 2, 10, 1000):
        s = oracle.adamw_scalars(1e-3, 0.9, 0.95, 1e-8, 0.1, t)
        assert s.b1 == np.float32(0.9) and s.b2 == np.float32(0.95)
        assert s.a1 == np.float32(1 - 0.9) and s.a2 == np.float32(1 - 0.95)
        assert s.eps == np.float32(1e-8)
        assert s.sigma == np.float32(1e-3 * math.sqrt(1 - 0.95 ** t) / (1 - 0.9 ** t))
        assert s.delta == np.float32(1 - 1e-3 * 0.1)
    # large t: corrections vanish, step size -> lr
    s = oracle.adamw_scalars(1e-3, 0.9, 0.95, 1e-8, 0.1, 100000)
    assert s.sigma == np.float32(1e-3)


# ------------------------------------------------------------------ (d)
def _exact_run(N, W, steps, grads_fn, master_full, hp_fn):
    """Exact-rational re-evaluation of every rank's step (softfloat)."""
    F32, F64 = sf.F32, sf.F64
    st = {r: None for r in range(W)}
    for r in range(W):
        b, e = shard_range(N, W, r)
        st[r] = dict(p=[sf.from_f32(x) for x in master_full[b:e]],
                     m=[sf.Fraction(0)] * (e - b), v=[sf.Fraction(0)] * (e - b), bf=None, info=[])
    for t in range(1, steps + 1):
        G = grads_fn(t)
        hp = hp_fn(t)
        gs, part = {}, []
        for r in range(W):
            b, e = shard_range(N, W, r)
            gr = []
            for i in range(b, e):
                s = sf.from_bf16_bits(G[0][i])
                for w in range(1, W):
                    s = sf.add(s, sf.from_bf16_bits(G[w][i]))
                gr.append(sf.div(s, sf.Fraction(W)))
            gs[r] = gr
            q = sf.Fraction(0)
            for x in gr:                  # one block: shard < 65536
                q = sf.add(q, x * x, F64)  # square exact in fp64
            part.append(q)
        tot = sf.Fraction(0)
        for q in part:
            tot = sf.add(tot, q, F64)
        norm = sf.sqrt(tot, F64)
        clip = norm > sf.Fraction(hp["max_norm"])
        coef = sf.rnd(sf.div(sf.Fraction(hp["max_norm"]), norm, F64), F32) if clip else None
        # scalars: doubles from Python floats, each op rounded to fp64, then to fp32
        lr, b1, b2 = sf.Fraction(hp["lr"]), hp["beta1"], hp["beta2"]
        bc1 = sf.sub(sf.Fraction(1), sf.Fraction(b1 ** t), F64)
        bc2 = sf.sub(sf.Fraction(1), sf.Fraction(b2 ** t), F64)
        sigma = sf.rnd(sf.div(sf.mul(lr, sf.sqrt(bc2, F64), F64), bc1, F64), F32)
        delta = sf.rnd(sf.sub(sf.Fraction(1), sf.mul(lr, sf.Fraction(hp["weight_decay"]), F64), F64), F32)
        B1, B2 = sf.rnd(sf.Fraction(b1)), sf.rnd(sf.Fraction(b2))
        A1 = sf.rnd(sf.sub(sf.Fraction(1), sf.Fraction(b1), F64))
        A2 = sf.rnd(sf.sub(sf.Fraction(1), sf.Fraction(b2), F64))
        EPS = sf.rnd(sf.Fraction(hp["eps"]))
        for r in range(W):
            S = st[r]
            for k, g in enumerate(gs[r]):
                if clip:
                    g = sf.mul(g, coef)
                m = sf.add(sf.mul(B1, S["m"][k]), sf.mul(A1, g))
                v = sf.add(sf.mul(B2, S["v"][k]), sf.mul(A2, sf.mul(g, g)))
                d = sf.add(sf.sqrt(v), EPS)
                q = sf.div(m, d)
                p = sf.sub(S["p"][k], sf.mul(sigma, q))
                p = sf.mul(p, delta)
                S["m"][k], S["v"][k], S["p"][k] = m, v, p
            S["bf"] = [sf.to_bf16_bits(p) for p in S["p"]]
            S["info"].append((norm, clip, coef))
    return st


def _special_grads(G, rng):
    """Sprinkle special bf16 values into small replica gradients."""
    specials = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x4000, 0x3C00]
    for g in G:
        idx = rng.choice(g.size, size=min(3, g.size), replace=False)
        g[idx] = rng.choice(specials, size=idx.size).astype(np.uint16)
    return G


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 64])
def test_oracle_matches_exact_rational(W):
    N = 16 * W
    steps = 10
    seed = 0xD00D + W
    rng = np.random.default_rng(W)
    cache = {}

    def grads_fn(t):
        if t not in cache:
            sigma = [1e-3, 1.0, 3e-2][t % 3]     # t%3==1 gives a norm above max_norm
            G = synth_grads(seed, t, W, N, sigma, outlier_pct=5)
            cache[t] = _special_grads(G, rng)
        return cache[t]

    master = synth.f32(N, synth.master_key(seed), 0, 0.02)
    master[0] = np.float32(1e-40)                  # a subnormal master value
    states = oracle_run(N, W, steps, grads_fn, master, lambda t: hp_at(t))
    exact = _exact_run(N, W, steps, grads_fn, master, lambda t: hp_at(t))
    clipped = 0
    for r in range(W):
        o, x = states[r], exact[r]
        for k in range(o.master.size):
            assert o.master[k] == np.float32(float(x["p"][k])), (r, k)
            assert o.m[k] == np.float32(float(x["m"][k])), (r, k)
            assert o.v[k] == np.float32(float(x["v"][k])), (r, k)
            assert int(o.param[k]) == x["bf"][k] or (o.param[k] & 0x7FFF) == 0 == (x["bf"][k] & 0x7FFF)
        for info, (norm, clip, coef) in zip(o.infos, x["info"]):
            assert info.norm == float(norm)
            assert info.clip == clip
            clipped += int(clip)
            if clip:
                assert info.coef == np.float32(float(coef))
    assert clipped > 0


# ------------------------------------------------------------------ invariants
def test_norm_scales_by_power_of_two():
    W, N = 3, 3 * 5000
    G = synth_grads(0xABC, 1, W, N, 1e-2)
    g = oracle.shard_reduce(G)
    q = oracle.sumsq(g)
    G2 = [oracle.f32_to_bf16(oracle.bf16_to_f32(x) * np.float32(2.0 ** 5)) for x in G]
    q2 = oracle.sumsq(oracle.shard_reduce(G2))
    assert q2 == q * 4.0 ** 5
    assert math.sqrt(q2) == math.sqrt(q) * 2.0 ** 5


def test_clip_brings_norm_to_max_norm():
    W, N = 4, 4 * 40000
    G = synth_grads(0xC11, 1, W, N, 1.0)
    g = oracle.shard_reduce(G)
    norm = math.sqrt(oracle.sumsq(g))
    assert norm > 1.0
    clip, c = oracle.clip_coef(norm, 1.0)
    assert clip
    gc = g * c
    assert abs(math.sqrt(float(np.sum(gc.astype(np.float64) ** 2))) - 1.0) < 1e-6
    # exactly at the threshold: no clip (strict test)
    assert oracle.clip_coef(1.0, 1.0)[0] is False
    assert oracle.clip_coef(float("nan"), 1.0)[0] is False
    clip, c = oracle.clip_coef(float("inf"), 1.0)
    assert clip and c == 0.0
    assert oracle.clip_coef(1e30, float("inf"))[0] is False


def test_w1_reduce_is_identity_and_sum_is_sequential():
    x = synth.bf16(100000, 123, 0, 1.0, 3)
    assert np.array_equal(oracle.shard_reduce([x]), oracle.bf16_to_f32(x))
    # three replicas whose order matters in fp32: (big + 1) - big
    big = _bf16_of([2.0 ** 30])
    one = _bf16_of([1.0])
    nbig = _bf16_of([-(2.0 ** 30)])
    assert oracle.shard_reduce([big, one, nbig], average=False)[0] == 0.0
    assert oracle.shard_reduce([big, nbig, one], average=False)[0] == 1.0


def test_sumsq_streaming_and_blocks():
    g = synth.f32(3 * 65536 + 123, 77, 0, 1.0)
    whole = oracle.sumsq(g)
    tot = 0.0
    for lo in range(0, g.size, 65536):
        tot = oracle.sumsq(g[lo:lo + 65536], tot)
    assert tot == whole
    # sequential within each block, then the block sums in order
    ref = 0.0
    for lo in range(0, g.size, 65536):
        s = 0.0
        for x in g[lo:lo + 65536].astype(np.float64).tolist():
            s = s + x * x
        ref = ref + s
    assert ref == whole


def test_zero1_equals_ddp_on_small_flat():
    """Concatenating all W ranks' updated shards equals one non-sharded step on
    the all-reduced average (reduce-scatter + all-gather = all-reduce)."""
    N, W, steps = 4 * 8192 + 8, 4, 4
    seed = 0x5EED
    master = synth.f32(N, synth.master_key(seed), 0, 0.02)
    cache = {}

    def grads_fn(t):
        if t not in cache:
            cache[t] = synth_grads(seed, t, W, N, 1e-2 if t != 2 else 1.0)
        return cache[t]

    sharded = oracle_run(N, W, steps, grads_fn, master, lambda t: hp_at(t))
    # non-sharded: one "rank" owning all N with the W replicas as input
    from tests.oracle_sim import RankState
    full = RankState(master)
    for t in range(1, steps + 1):
        G = grads_fn(t)
        rs = np.zeros(1)
        oracle.step(G, full.master, full.m, full.v, full.param, hp_at(t), rs, 0)
        full.infos.append(None)
    cat = lambda f: np.concatenate([getattr(sharded[r], f) for r in range(W)])
    for f in ("master", "m", "v", "param"):
        assert np.array_equal(cat(f), getattr(full, f)), f


def test_zero_memory_accounting():
    g = _kv("zero_memory_7p5b_64gpu.txt")
    for stage in range(4):
        b = oracle.zero_bytes_per_gpu(g["psi"], g["K"], g["n_d"], stage) / 1e9
        assert round(b, 1) == g[f"stage{stage}"]
    assert oracle.zero_bytes_per_gpu(7.5e9, 12, 64, 1) / 1e9 == pytest.approx(31.40625)
    assert oracle.zero_bytes_per_gpu(7.5e9, 12, 64, 3) / 1e9 == pytest.approx(1.875)
    # 16 B/param for full AdamW: 7B params -> 112 GB
    assert oracle.zero_bytes_per_gpu(7e9, 12, 1, 0) / 1e9 == pytest.approx(112.0)


def test_fp_env_keeps_subnormals():
    assert oracle.fp_env_ok()
    g = _bf16_of([2.0 ** -130])
    out = oracle.shard_reduce([g, g], average=True)
    assert out[0] == np.float32(2.0 ** -130)


# ------------------------------------------------------------------ RNE
def test_rne_against_torch_bfloat16_all_patterns():
    """The oracle's fp32->bf16 rounding against torch's bfloat16 conversion over
    every one of the 2^32 binary32 bit patterns (NaNs: both must be NaN)."""
    torch = pytest.importorskip("torch")
    chunk = 1 << 26
    for lo in range(0, 1 << 32, chunk):
        bits = np.arange(lo, lo + chunk, dtype=np.uint32)
        x = bits.view(np.float32)
        ours = oracle.f32_to_bf16(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        assert np.array_equal(ours[~nan], ref[~nan]), hex(lo)
        assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)
        # sign kept on NaN
        assert np.array_equal(ours[nan] >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_rne_against_softfloat_samples():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0x3F808000, 0x3F818000, 0x7F7FFFFF, 0x7F7F8000, 0x00008000, 0x00018000, 0x80000000, 0x7F800000]
    x = bits.view(np.float32)
    ours = oracle.f32_to_bf16(x)
    for xi, oi in zip(x.tolist(), ours.tolist()):
        if math.isnan(xi):
            continue
        ref = sf.to_bf16_bits(sf.from_f32(xi))
        if xi < 0 or (xi == 0 and struct.pack("<f", xi)[3] & 0x80):
            ref |= 0x8000
        assert oi == ref, (xi, hex(oi), hex(ref))


# ------------------------------------------------------------------ compatibility variants
def test_decay_first_closed_form_and_gap():
    """Decay-first order (the order the page attributes to torch.optim.AdamW):
    under a constant gradient p_t = p_{t-1}*(1-lr*wd) - u_t, and over many
    steps the two orders drift apart by the sum of sigma_t*|q_t|*lr*wd (the
    page's 'order lr^2*lambda per step'), here on the quadratic f(x) = x^2/2."""
    lr, wd = 1e-3, 0.1
    gval = 2.0 ** -7
    g = _bf16_of([gval])
    p = np.array([0.25], np.float32)
    m = np.zeros(1, np.float32)
    v = np.zeros(1, np.float32)
    p64 = 0.25
    for t in range(1, 11):
        oracle.step([g], p, m, v, oracle.f32_to_bf16(p), hp_at(t, max_norm=math.inf), np.zeros(1), 0,
                    variant=oracle.DECAY_FIRST)
        bc2 = 1 - 0.95 ** t
        u = lr * gval * math.sqrt(bc2) / (math.sqrt(bc2) * gval + 1e-8)
        p64 = p64 * (1 - lr * wd) - u
        assert abs(float(p[0]) - p64) <= 1e-6 * abs(p64)
    # quadratic: gradient = x (fed as an exact bf16 value each step), both orders
    xs = {}
    for var in (0, oracle.DECAY_FIRST):
        x = np.array([1.0], np.float32)
        m = np.zeros(1, np.float32)
        v = np.zeros(1, np.float32)
        bound = 0.0
        for t in range(1, 101):
            gb = oracle.f32_to_bf16(x.copy())
            s = oracle.adamw_scalars(lr, 0.9, 0.95, 1e-8, wd, t)
            # |m/(sqrt(v)+eps)| stays below ~3 for Adam with these betas
            bound += float(s.sigma) * 3.0 * lr * wd * (1 + abs(float(x[0])))
            oracle.step([gb], x, m, v, oracle.f32_to_bf16(x), hp_at(t, max_norm=math.inf), np.zeros(1), 0,
                        variant=var)
        xs[var] = float(x[0])
    gap = abs(xs[0] - xs[oracle.DECAY_FIRST])
    assert 0 < gap <= bound + 1e-6


def test_decay_order_gap_has_the_pages_order_of_magnitude():
    """The page runs its AdamW (update, then decay) against torch's (decay,
    then update) for 100 steps on a quadratic and reports a largest difference
    of 8.4e-4, which it attributes to the order alone (a term of order
    lr^2*lambda per step).  The page gives neither the quadratic nor the
    hyper-parameters, so the exact figure stays unpinned; under the reading
    f(x) = x^2/2 from x = 1, lr = 1e-2, lambda = 0.1, betas (0.9, 0.999),
    eps = 1e-8 the two orders end up differing by the same order of magnitude
    (about 4.6e-4), and the gap grows with lr^2*lambda as the page says."""
    def run(lr, wd, variant):
        x = np.array([1.0], np.float32)
        m = np.zeros(1, np.float32)
        v = np.zeros(1, np.float32)
        out = []
        for t in range(1, 101):
            hp = dict(lr=lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, max_norm=math.inf, step=t)
            oracle.step([oracle.f32_to_bf16(x.copy())], x, m, v, oracle.f32_to_bf16(x), hp, np.zeros(1), 0,
                        variant=variant)
            out.append(float(x[0]))
        return np.array(out)

    def gap(lr, wd):
        return float(np.max(np.abs(run(lr, wd, 0) - run(lr, wd, oracle.DECAY_FIRST))))

    g = gap(1e-2, 0.1)
    assert 1e-4 < g < 1e-2 and abs(math.log10(g) - math.log10(8.4e-4)) < 0.5, g
    # scaling: ten times lambda, or about ten times lr^2, gives a gap ten times larger or so
    assert 5 < gap(1e-2, 0.1) / gap(1e-2, 0.01) < 20
    assert 3 < gap(1e-2, 0.1) / gap(3e-3, 0.1) < 30


@pytest.mark.parametrize("order", ["update_then_decay", "decay_first"])
@pytest.mark.parametrize("lr,b2,eps", [(1e-2, 0.99, 1e-6), (1e-3, 0.95, 1e-8)])
def test_adamw_against_torch_optim_adamw(order, lr, b2, eps):
    """The oracle's AdamW against torch.optim.AdamW (the library routine, run
    in float64 as the exact reference) over 30 steps of random bf16 gradients
    spanning four decades.  Two mathematical identities map the page's step
    onto torch's: torch adds eps to sqrt(v)/sqrt(1-beta2^t), so the folded
    form's eps equals torch's eps times sqrt(1-beta2^t); and the page's order
    p <- (p - sigma*q)*delta equals torch's decay-first step run with learning
    rate lr*delta and weight decay wd/delta.  What remains is the fp32 master's
    own rounding: per step, delta rounded to binary32, the product and the
    difference (up to 1.5 ulp of |p|) and a few ulps of the step itself; the
    bound below allows 2 ulps of |p| and 2^-22 * 8 lr per step and element."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0xADA + int(1e4 * lr))
    n, T, b1, wd = 4096, 30, 0.9, 0.1
    p0 = rng.normal(0, 0.5, n).astype(np.float32)
    x = p0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    delta = 1.0 - lr * wd
    variant = oracle.DECAY_FIRST if order == "decay_first" else 0
    t_lr, t_wd = (lr, wd) if variant else (lr * delta, wd / delta)
    tp = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=t_lr, betas=(b1, b2), eps=eps, weight_decay=t_wd, foreach=False)
    pmax = np.abs(p0).astype(np.float64)
    for t in range(1, T + 1):
        gb = oracle.f32_to_bf16(rng.normal(0, 1, n).astype(np.float32) * np.float32(10.0 ** -rng.integers(0, 4)))
        hp = dict(lr=lr, beta1=b1, beta2=b2, eps=eps * math.sqrt(1 - b2 ** t), weight_decay=wd,
                  max_norm=math.inf, step=t)
        oracle.step([gb], x, m, v, oracle.f32_to_bf16(x), hp, np.zeros(1), 0, variant=variant)
        tp.grad = torch.tensor(oracle.bf16_to_f32(gb).astype(np.float64))
        opt.step()
        ref = tp.detach().numpy()
        pmax = np.maximum(pmax, np.abs(ref))
        bound = t * 2.0 ** -22 * (pmax + 8 * lr)
        err = np.abs(x.astype(np.float64) - ref)
        assert (err <= bound).all(), (order, t, float((err / bound).max()))
    st = opt.state[tp]
    # the second moment is positive: a plain relative bound holds for it
    vv = st["exp_avg_sq"].numpy()
    assert np.max(np.abs(v - vv) / vv) < 1e-5
    # the first moment, in units of the gradient scale it averages
    assert np.max(np.abs(m - st["exp_avg"].numpy()) / np.sqrt(vv)) < 1e-5


def test_torch_clip_convention_against_torch():
    """The torch clip variant reproduces torch.nn.utils.clip_grad_norm_'s
    coefficient (max_norm / (norm + 1e-6), clamped at 1; fp64 gradients)."""
    torch = pytest.importorskip("torch")
    for norm_target, max_norm in [(1.25, 1.0), (0.5, 1.0), (1.0, 1.0), (3.0e5, 2.0)]:
        x = torch.zeros(3, dtype=torch.float64)
        x[0] = 1.0
        x[1] = math.sqrt(norm_target ** 2 - 1.0) if norm_target > 1 else 0.0
        if norm_target <= 1:
            x[0] = norm_target
        nrm = float(torch.linalg.vector_norm(x))
        p = torch.nn.Parameter(torch.zeros(3, dtype=torch.float64))
        p.grad = x.clone()
        torch.nn.utils.clip_grad_norm_([p], max_norm)
        torch_coef = float(p.grad[0] / x[0])
        clip, coef = oracle.clip_coef_eps(nrm, max_norm)
        assert coef == np.float32(torch_coef), (norm_target, coef, torch_coef)
        assert clip == (torch_coef < 1.0)
    # at the threshold the torch convention clips (slightly), the pages' does not
    assert oracle.clip_coef_eps(1.0, 1.0)[0] and not oracle.clip_coef(1.0, 1.0)[0]


def test_g_bf16_variant_is_a_step_on_the_rounded_gradient():
    """Rounding the reduced gradient to bf16 before the norm and the update is
    the same as one plain step whose single replica is that bf16 gradient."""
    W, N = 5, 20000
    G = synth_grads(0xB16, 1, W, N, 0.3, outlier_pct=2)
    gb = oracle.f32_to_bf16(oracle.shard_reduce(G))
    assert np.array_equal(oracle.bf16_to_f32(gb), oracle.round_to_bf16(oracle.shard_reduce(G)))
    master = synth.f32(N, synth.master_key(3), 0, 0.02)
    a = [master.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32), np.zeros(N, np.uint16)]
    b = [master.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32), np.zeros(N, np.uint16)]
    ia = oracle.step(G, *a, hp_at(1), np.zeros(1), 0, variant=oracle.G_BF16)
    ib = oracle.step([gb], *b, hp_at(1), np.zeros(1), 0)
    assert ia.norm == ib.norm and ia.coef == ib.coef and ia.clip
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # and it differs from the fp32-gradient step
    c = [master.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32), np.zeros(N, np.uint16)]
    oracle.step(G, *c, hp_at(1), np.zeros(1), 0)
    assert not np.array_equal(c[0], a[0])


def test_zero_gradient_step_is_pure_decay():
    """Degenerate case: every replica's gradient is zero.  The norm is 0, so
    nothing is clipped; m and v stay exactly 0 (b*0 + a*0), the Adam term is
    0/(sqrt(0)+eps) = 0, and the master is only decayed: p*delta, one rounding.
    With eps = 0 the term is 0/0: NaN by IEEE, which the oracle must carry."""
    rng = np.random.default_rng(11)
    N, W = 1000, 3
    master0 = rng.standard_normal(N).astype(np.float32)
    zero = [np.zeros(N, np.uint16) for _ in range(W)]
    for t in (1, 2, 7):
        master, m, v = master0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
        param = np.zeros(N, np.uint16)
        rs = np.zeros(1)
        info = oracle.step(zero, master, m, v, param, hp_at(t), rs, 0)
        assert info.norm == 0.0 and not info.clip and info.coef == np.float32(1.0)
        assert not m.any() and not v.any()
        delta = np.float32(1.0 - 1e-3 * 0.1)
        assert np.array_equal(master, master0 * delta)
        assert np.array_equal(param, oracle.f32_to_bf16(master0 * delta))
    # negative zeros in the gradient behave like +0 (the average of -0 and +0 is +0 or -0; g*g is +0)
    negz = [np.full(N, 0x8000, np.uint16) for _ in range(W)]
    master, m, v = master0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
    oracle.step(negz, master, m, v, np.zeros(N, np.uint16), hp_at(1), np.zeros(1), 0)
    assert np.array_equal(master, master0 * np.float32(1.0 - 1e-3 * 0.1))
    # eps = 0: 0/0
    master, m, v = master0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
    oracle.step(zero, master, m, v, np.zeros(N, np.uint16), hp_at(1, eps=0.0), np.zeros(1), 0)
    assert np.isnan(master).all()
