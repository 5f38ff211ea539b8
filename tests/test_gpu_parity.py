"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, on seeded inputs that span several tiles, ragged tails, misaligned
starts, special values and every rank.  Floating-point results must be
bit-identical to the oracle (the operation sequence is the same); norms, whose
fp64 partial sums are added in a different order, must agree to 1e-12
relative, and the clip decision and coefficient must be identical."""
from __future__ import annotations

import math
import zlib

import numpy as np
import pytest

import oracle
import synth
import zero_sharded_mixed_zero1_amd as z
from synth.workloads import shard_range
from tests.gpu_util import (MtaShard, assert_bf16_equal, assert_f32_equal, rel_close, to_dev_u16,
                            to_np_u16, torch_cuda, ws_tensor)

pytestmark = pytest.mark.gpu

NORM_TOL = 1e-12


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return torch, dev


def hp_at(t, **kw):
    d = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, step=t)
    d.update(kw)
    return d


SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x4000,
                     0x3C00, 0x7F7F, 0x00FF], dtype=np.uint16)


def replicas(seed, t, W, N, sigma, outlier_pct=0, specials=0, rng=None):
    G = [synth.bf16(N, synth.grad_key(seed, t, w), 0, sigma, outlier_pct) for w in range(W)]
    if specials and N:
        rng = rng or np.random.default_rng(seed + t)
        for g in G:
            idx = rng.choice(N, size=min(specials, N), replace=False)
            g[idx] = rng.choice(SPECIALS, size=idx.size)
    return G


# ---------------------------------------------------------------- input generator
def test_synth_gpu_matches_cpu(env):
    torch, dev = env
    for n, i0, sigma, pct in [(1, 0, 1e-3, 0), (1000003, 17, 1e-2, 1), (4096, 1 << 40, 0.02, 0),
                              (333333, 5_000_000_000, 1e-3, 7)]:
        k = synth.grad_key(0xABCDEF, 3, 5)
        tb = torch.empty(n, dtype=torch.int16, device=dev)
        synth.fill_bf16_(tb, k, i0, sigma, pct)
        tf = torch.empty(n, dtype=torch.float32, device=dev)
        synth.fill_f32_(tf, k, i0, sigma, pct)
        torch.cuda.synchronize()
        assert np.array_equal(to_np_u16(tb), synth.bf16(n, k, i0, sigma, pct))
        assert np.array_equal(tf.cpu().numpy().view(np.uint32), synth.f32(n, k, i0, sigma, pct).view(np.uint32))


# ---------------------------------------------------------------- reduce + norm
LENGTHS = [0, 1, 7, 8, 9, 2047, 2048, 2049, 16384 + 5, 3 * 65536 + 13]


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 64])
def test_shard_reduce_parity(env, W):
    torch, dev = env
    ws = ws_tensor(torch, z.workspace_bytes(1 << 20, W), dev)
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    for length in LENGTHS:
        for offset in (0, 1, 3, 8):
            if W == 64 and offset not in (0, 3):
                continue
            N = offset + length + 5
            G = replicas(1000 + W, length + offset, W, N, 0.5, outlier_pct=2, specials=3)
            gd = [to_dev_u16(torch, g, dev) for g in G]
            for flags in (0, z.SUM_ONLY):
                gout = torch.full((length + 4,), float("nan"), dtype=torch.float32, device=dev)
                go = gout[1:] if offset == 3 else gout       # also a misaligned output
                z.shard_reduce(gd, offset, length, g_out=go, sumsq_out=sumsq, flags=flags, ws=ws)
                torch.cuda.synchronize()
                exp = oracle.shard_reduce([g[offset:offset + length] for g in G],
                                          average=not (flags & z.SUM_ONLY))
                got = go[:length].cpu().numpy()
                assert_f32_equal(got, exp, f"g W={W} len={length} off={offset} flags={flags}")
                assert np.isnan(go[length:].cpu().numpy()).all(), "wrote past the end"
                q = float(sumsq.item())
                assert rel_close(q, oracle.sumsq(exp), NORM_TOL), (W, length, offset, q)
            # norm only (no g_out) gives the same partial bit for bit
            s2 = torch.zeros(1, dtype=torch.float64, device=dev)
            z.shard_reduce(gd, offset, length, sumsq_out=s2, ws=ws)
            z.shard_reduce(gd, offset, length, g_out=gout, sumsq_out=sumsq, ws=ws)
            torch.cuda.synchronize()
            assert s2.item() == sumsq.item()


def test_grad_norm_parity(env):
    torch, dev = env
    ws = ws_tensor(torch, z.workspace_bytes(1 << 22, 1), dev)
    out = torch.zeros(1, dtype=torch.float64, device=dev)
    for n in (0, 1, 9, 2048, 65536 * 5 + 3, 3_000_001):
        x = synth.f32(n + 1, synth.key(77, n), 0, 3.0, 1)
        x[:: max(1, n // 7)] = np.float32(1e-42)     # subnormals
        t = torch.from_numpy(x).to(dev)
        for view in (t[:n], t[1:n + 1]):
            z.grad_norm(view, n, out, ws=ws)
            torch.cuda.synchronize()
            exp = oracle.sumsq(view.cpu().numpy())
            assert rel_close(out.item(), exp, NORM_TOL), (n, out.item(), exp)
    # the fp32 g of shard_reduce and its partial agree with grad_norm over that g
    G = replicas(5, 1, 3, 100_000, 1e-2)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    g = torch.empty(100_000, dtype=torch.float32, device=dev)
    s1 = torch.zeros(1, dtype=torch.float64, device=dev)
    z.shard_reduce(gd, 0, 100_000, g_out=g, sumsq_out=s1, ws=ws)
    z.grad_norm(g, 100_000, out, ws=ws)
    torch.cuda.synchronize()
    assert s1.item() == out.item()


# ---------------------------------------------------------------- flat AdamW
@pytest.mark.parametrize("mv_bf16", [False, True])
@pytest.mark.parametrize("source", ["g", "recompute3", "recompute8"])
def test_adamw_step_flat_parity(env, mv_bf16, source):
    torch, dev = env
    W = {"g": 4, "recompute3": 3, "recompute8": 8}[source]
    for length, offset, max_norm, t0 in [(1, 0, 1.0, 1), (2049, 0, 1.0, 1), (65536 * 3 + 7, 0, 1e9, 2),
                                         (4103, 5, 1.0, 999), (20000, 8, math.inf, 1)]:
        seed = zlib.crc32(f"{length}/{offset}/{source}".encode()) & 0xFFFFFF
        N = offset + length
        master0 = synth.f32(N, synth.master_key(seed), 0, 0.02)[offset:]
        k = min(3, length)
        master0[:k] = np.array([1e-40, -0.0, 3e38], dtype=np.float32)[:k]
        mvd = torch.int16 if mv_bf16 else torch.float32
        npmv = np.uint16 if mv_bf16 else np.float32
        gm = torch.from_numpy(master0.copy()).to(dev)
        gmm = torch.zeros(length, dtype=mvd, device=dev)
        gvv = torch.zeros(length, dtype=mvd, device=dev)
        gp = torch.zeros(length + 1, dtype=torch.int16, device=dev)[1:] if offset == 5 else \
            torch.zeros(length, dtype=torch.int16, device=dev)
        om, ov = np.zeros(length, npmv), np.zeros(length, npmv)
        omaster, oparam = master0.copy(), np.zeros(length, np.uint16)
        ws = ws_tensor(torch, z.workspace_bytes(length, W), dev)
        info = torch.zeros(4, dtype=torch.float64, device=dev)
        gbuf = torch.empty(length, dtype=torch.float32, device=dev)
        for t in range(t0, t0 + 3):
            G = replicas(seed, t, W, N, 0.05 if t % 2 else 0.001, outlier_pct=1, specials=2)
            sl = [g[offset:] for g in G]
            hp = hp_at(t, max_norm=max_norm)
            other = np.array([0.0, 0.37, 0.0], dtype=np.float64)     # three "ranks"; we are rank 0
            rs = other.copy()
            oinfo = oracle.step(sl, omaster, om, ov, oparam, hp, rs, 0)
            gd = [to_dev_u16(torch, g, dev) for g in G]
            rsd = torch.from_numpy(rs).to(dev)                      # includes this rank's oracle partial
            if source == "g":
                sq = torch.zeros(1, dtype=torch.float64, device=dev)
                z.shard_reduce(gd, offset, length, g_out=gbuf, sumsq_out=sq, ws=ws)
                torch.cuda.synchronize()
                assert rel_close(sq.item(), rs[0], NORM_TOL)
                z.adamw_step(gbuf, None, 0, length, gm, gmm, gvv, gp, hp, rsd, 3,
                             flags=z.MV_BF16 if mv_bf16 else 0, info_out=info)
            else:
                z.adamw_step(None, gd, offset, length, gm, gmm, gvv, gp, hp, rsd, 3,
                             flags=z.MV_BF16 if mv_bf16 else 0, info_out=info)
            torch.cuda.synchronize()
            ni = info.cpu().numpy()
            assert ni[1] == oinfo.norm                        # same partials in, same norm out
            iw = info.cpu().numpy().view(np.int32)
            assert bool(iw[5]) == oinfo.clip
            assert info.cpu().numpy()[2:3].view(np.float32)[0] == oinfo.coef
        what = f"len={length} off={offset} src={source} bf16mv={mv_bf16}"
        assert_f32_equal(gm.cpu().numpy(), omaster, "master " + what)
        if mv_bf16:
            assert_bf16_equal(to_np_u16(gmm), om, "m " + what)
            assert_bf16_equal(to_np_u16(gvv), ov, "v " + what)
        else:
            assert_f32_equal(gmm.cpu().numpy(), om, "m " + what)
            assert_f32_equal(gvv.cpu().numpy(), ov, "v " + what)
        assert_bf16_equal(to_np_u16(gp), oparam, "param " + what)


@pytest.mark.parametrize("case", range(30))
def test_flat_entry_points_random(env, case):
    """Seeded random calls of the flat entry points, two steps each:
    zero1_shard_reduce (g and this rank's sum of squares) then
    zero1_adamw_step with that g, or zero1_adamw_step recomputing g from the
    slices (with zero1_shard_reduce giving the sum of squares alone); W from 1
    to 128, lengths from 0 to 200,000 at any offset into the replica buffers,
    state buffers on or off 16-byte boundaries, sum or average, fp32 or bf16
    moments, compatibility variants, t up to 2000.  State bit for bit, the
    partial to 1e-12, the clip decision and coefficient identical."""
    torch, dev = env
    rng = np.random.default_rng(0xF1A7 + case)
    W = int(rng.integers(1, 129))
    length = int(rng.choice([0, 1, 2047, 2048, int(rng.integers(1, 200001)), int(rng.integers(1, 200001))]))
    offset = int(rng.integers(0, 9))
    from_g = bool(rng.integers(0, 2))
    mv_bf16 = bool(rng.integers(0, 2))
    sum_only = bool(rng.integers(0, 4) == 0)
    variant = int(rng.choice([0, 0, oracle.DECAY_FIRST, oracle.CLIP_EPS, oracle.G_BF16,
                              oracle.DECAY_FIRST | oracle.G_BF16]))
    t0 = int(rng.integers(1, 2001))
    max_norm = float(rng.choice([1.0, 0.05, math.inf]))
    sigma = float(rng.choice([1e-4, 1e-2, 0.3]))
    skew = int(rng.integers(0, 2))            # 1: state buffers one element past an aligned start
    n_ranks = int(rng.integers(1, 5))        # this rank is rank 0
    seed = 0xF1B0 + case
    N = offset + length
    master0 = synth.f32(N + 1, synth.master_key(seed), 0, 0.02)[offset:offset + length].copy()
    mvd, npmv = (torch.int16, np.uint16) if mv_bf16 else (torch.float32, np.float32)

    def buf(n, dt):
        return torch.zeros(n + skew, dtype=dt, device=dev)[skew:]

    gm, gmm, gvv, gp = buf(length, torch.float32), buf(length, mvd), buf(length, mvd), buf(length, torch.int16)
    gm.copy_(torch.from_numpy(master0))
    om, ov = np.zeros(length, npmv), np.zeros(length, npmv)
    omaster, oparam = master0.copy(), np.zeros(length, np.uint16)
    ws = ws_tensor(torch, z.workspace_bytes(length, W), dev)
    gbuf = torch.empty(max(length, 1), dtype=torch.float32, device=dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    sq = torch.zeros(1, dtype=torch.float64, device=dev)
    red_flags = (z.SUM_ONLY if sum_only else 0) | (z.G_BF16 if variant & oracle.G_BF16 else 0)
    upd_flags = (z.MV_BF16 if mv_bf16 else 0) | lib_flags(variant & (oracle.DECAY_FIRST | oracle.CLIP_EPS))
    what = (f"case={case} W={W} len={length} off={offset} from_g={from_g} bf16mv={mv_bf16} sum_only={sum_only} "
            f"variant={variant} skew={skew} ranks={n_ranks} t0={t0}")
    for t in (t0, t0 + 1):
        G = replicas(seed, t, W, N + 1, sigma, outlier_pct=1, specials=3, rng=rng)   # one element past the range
        hp = hp_at(t, max_norm=max_norm)
        rs = np.concatenate([[0.0], rng.random(n_ranks - 1) * 3.0])
        oinfo = oracle.step([g[offset:offset + length] for g in G], omaster, om, ov, oparam, hp, rs, 0,
                            average=not sum_only, variant=variant)
        gd = [to_dev_u16(torch, g, dev) for g in G]
        z.shard_reduce(gd, offset, length, g_out=gbuf if from_g else None, sumsq_out=sq, flags=red_flags, ws=ws)
        torch.cuda.synchronize()
        assert rel_close(sq.item(), rs[0], NORM_TOL), (what, sq.item(), rs[0])
        rsd = torch.from_numpy(rs).to(dev)                 # the oracle's partials: the norms agree bit for bit
        if from_g:
            z.adamw_step(gbuf, None, 0, length, gm, gmm, gvv, gp, hp, rsd, n_ranks, flags=upd_flags, info_out=info)
        else:
            z.adamw_step(None, gd, offset, length, gm, gmm, gvv, gp, hp, rsd, n_ranks, flags=upd_flags | red_flags,
                         info_out=info)
        torch.cuda.synchronize()
        ni = info.cpu().numpy()
        assert ni[1] == oinfo.norm or (math.isnan(ni[1]) and math.isnan(oinfo.norm)), what
        assert bool(ni.view(np.int32)[5]) == oinfo.clip, what
        assert ni[2:3].view(np.float32)[0] == oinfo.coef or oinfo.coef != oinfo.coef, what
    assert_f32_equal(gm.cpu().numpy(), omaster, "master " + what)
    if mv_bf16:
        assert_bf16_equal(to_np_u16(gmm), om, "m " + what)
        assert_bf16_equal(to_np_u16(gvv), ov, "v " + what)
    else:
        assert_f32_equal(gmm.cpu().numpy(), om, "m " + what)
        assert_f32_equal(gvv.cpu().numpy(), ov, "v " + what)
    assert_bf16_equal(to_np_u16(gp), oparam, "param " + what)


# ---------------------------------------------------------------- multi-tensor apply
RAGGED = [3000, 17, 5000, 8, 2203, 1, 65536 + 3, 768, 8192 * 2, 40000]
# ragged against the 2048-element tiles but every piece 8-aligned, and a total
# that every W in the tests cuts into 8-aligned shards (what real tensor lists
# look like: the vector path end to end)
RAGGED8 = [3000, 16, 5000, 8, 2208, 8, 65536 + 8, 768, 8192 * 2, 40120]
assert sum(RAGGED8) % (8 * 24) == 0


VARIANT_FLAGS = {oracle.DECAY_FIRST: z.DECAY_FIRST, oracle.CLIP_EPS: z.CLIP_EPS, oracle.G_BF16: z.G_BF16}


def lib_flags(variant):
    return sum(f for v, f in VARIANT_FLAGS.items() if variant & v)


def run_mta_all_ranks(torch, dev, numels, W, steps, seed, flags, mv_bf16, flat_state, sigma_fn,
                      max_norm=1.0, ranks=None, variant=0, sum_only=False, hp_kw=None):
    N = sum(numels)
    ranks = list(range(W)) if ranks is None else ranks
    master_full = synth.f32(N, synth.master_key(seed), 0, 0.02)
    shards = {r: MtaShard(torch, dev, numels, W, r, master_full, mv_bf16, flat_state) for r in ranks}
    wss = {r: shards[r].workspace(flags) for r in ranks}
    from tests.oracle_sim import RankState
    ost = {r: RankState(master_full[slice(*shard_range(N, W, r))], mv_bf16) for r in ranks}
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    ws_r = ws_tensor(torch, z.workspace_bytes(N, W), dev)
    infos = torch.zeros((W, 4), dtype=torch.float64, device=dev)
    for t in range(1, steps + 1):
        G = replicas(seed, t, W, N, sigma_fn(t), outlier_pct=1)
        gd = [to_dev_u16(torch, g, dev) for g in G]
        part = np.zeros(W)
        for r in range(W):
            b, e = shard_range(N, W, r)
            gr = oracle.shard_reduce([g[b:e] for g in G], average=not sum_only)
            if variant & oracle.G_BF16:
                gr = oracle.round_to_bf16(gr)
            part[r] = oracle.sumsq(gr)
            # every rank's partial from the GPU (what the mid-step exchange would deliver)
            z.shard_reduce(gd, b, e - b, sumsq_out=rsd[r:r + 1], flags=lib_flags(variant) | (z.SUM_ONLY if sum_only else 0),
                           ws=ws_r)
        torch.cuda.synchronize()
        gpu_part = rsd.cpu().numpy().copy()
        for r in range(W):
            assert rel_close(gpu_part[r], part[r], NORM_TOL)
        hp = hp_at(t, max_norm=max_norm, **(hp_kw or {}))
        for r in ranks:
            b, e = shard_range(N, W, r)
            rs = part.copy()
            oi = oracle.step([g[b:e] for g in G], ost[r].master, ost[r].m, ost[r].v, ost[r].param, hp, rs, r,
                             average=not sum_only, variant=variant)
            rsd.copy_(torch.from_numpy(gpu_part))
            z.mta_step(gd, b, shards[r].plan, hp, rsd, W, r,
                       flags=flags | lib_flags(variant) | (z.SUM_ONLY if sum_only else 0), info_out=infos[r], ws=wss[r])
            torch.cuda.synchronize()
            ni = infos[r].cpu().numpy()
            assert rel_close(ni[1], oi.norm, NORM_TOL)
            assert bool(ni[2:4].view(np.int32)[1]) == oi.clip
            assert ni[2:3].view(np.float32)[0] == oi.coef
            assert rel_close(rsd[r].item(), part[r], NORM_TOL)
    for r in ranks:
        master, m, v, param = shards[r].gather()
        what = f"rank {r}/{W} flags={flags} bf16mv={mv_bf16} flat={flat_state} variant={variant}"
        assert_f32_equal(master, ost[r].master, "master " + what)
        if mv_bf16:
            assert_bf16_equal(m, ost[r].m, "m " + what)
            assert_bf16_equal(v, ost[r].v, "v " + what)
        else:
            assert_f32_equal(m, ost[r].m, "m " + what)
            assert_f32_equal(v, ost[r].v, "v " + what)
        assert_bf16_equal(param, ost[r].param, "param " + what)
        assert shards[r].untouched_outside(), "wrote outside the shard's pieces: " + what
    return shards, ost


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_mta_parity_ragged_all_ranks(env, W, design):
    torch, dev = env
    run_mta_all_ranks(torch, dev, RAGGED, W, 3, 0xA000 + W, design, False, True,
                      lambda t: [0.02, 1e-4, 0.3][t % 3])


@pytest.mark.parametrize("mv_bf16,flat_state", [(True, True), (False, False), (True, False)])
def test_mta_parity_state_layouts(env, mv_bf16, flat_state):
    torch, dev = env
    for design in (z.STORE_G, z.RECOMPUTE_G):
        run_mta_all_ranks(torch, dev, RAGGED, 4, 3, 0xB000, design, mv_bf16, flat_state,
                          lambda t: [0.02, 1e-4, 0.3][t % 3])


@pytest.mark.parametrize("W", [3, 8])
@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_mta_sum_only_parity(env, W, design):
    """ZERO1_SUM_ONLY (the reduce keeps the sum, no average) through the whole
    multi-tensor step on every design, every rank, against the oracle's
    unaveraged step."""
    torch, dev = env
    run_mta_all_ranks(torch, dev, RAGGED, W, 2, 0xD800 + W, design, False, True,
                      lambda t: 0.05, sum_only=True)


# Edge values of the hyper-parameters the boundary accepts: no moment memory
# (beta 0: m = g, v = g*g), no step (lr 0: sigma 0, decay factor 1), no decay,
# moments that forget almost nothing (bias corrections near 1e-6 at t = 1, so
# sigma is lr * 1e3), an eps that dominates sqrt(v), a large step, and a decay
# factor 1 - lr*wd that is negative.
DEGENERATE_HP = {
    "beta1=0": dict(beta1=0.0),
    "beta2=0": dict(beta2=0.0),
    "beta1=beta2=0": dict(beta1=0.0, beta2=0.0),
    "lr=0": dict(lr=0.0),
    "wd=0": dict(weight_decay=0.0),
    "beta=1-1e-6": dict(beta1=1.0 - 1e-6, beta2=1.0 - 1e-6),
    "eps=1": dict(eps=1.0),
    "lr=10": dict(lr=10.0, weight_decay=0.05),
    "decay factor -1": dict(lr=1.0, weight_decay=2.0),
}


@pytest.mark.parametrize("name", list(DEGENERATE_HP))
@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_degenerate_hyperparameters(env, name, design):
    """Every design on a ragged list, three steps, one rank (fp32 moments) and
    another (bf16 moments), bit-exact against the oracle."""
    torch, dev = env
    kw = DEGENERATE_HP[name]
    for r, mv_bf16 in ((1, False), (2, True)):
        run_mta_all_ranks(torch, dev, RAGGED, 3, 3, 0xDE00 + r, design, mv_bf16, True,
                          lambda t: [0.02, 1e-4, 0.3][t % 3], ranks=[r], hp_kw=kw)


@pytest.mark.parametrize("variant", [oracle.DECAY_FIRST, oracle.CLIP_EPS, oracle.G_BF16,
                                     oracle.DECAY_FIRST | oracle.CLIP_EPS | oracle.G_BF16])
@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_compat_variants_parity(env, variant, design):
    """Decay-first order, the torch clip convention and a bf16 reduced
    gradient (with bf16 moments), each against the oracle's variant, every
    rank, 3 steps, both step designs."""
    torch, dev = env
    run_mta_all_ranks(torch, dev, RAGGED8, 4, 3, 0xD000 + variant, design, variant == oracle.G_BF16, True,
                      lambda t: [0.02, 1e-4, 0.3][t % 3], variant=variant)


def test_compat_variants_flat_adamw(env):
    """The same variants through zero1_shard_reduce + zero1_adamw_step (g given,
    and g recomputed from the slices).  In step 2 max_norm equals that step's
    norm exactly: the pages' strict test does not clip, the torch convention
    (norm + 1e-6 in the denominator) does."""
    torch, dev = env
    W, N = 3, 70001
    for variant in (oracle.DECAY_FIRST, oracle.CLIP_EPS, oracle.G_BF16, 7):
        fl = lib_flags(variant)
        master0 = synth.f32(N, synth.master_key(77), 0, 0.02)
        for recompute in (False, True):
            gm = torch.from_numpy(master0.copy()).to(dev)
            gmm = torch.zeros(N, dtype=torch.float32, device=dev)
            gvv = torch.zeros(N, dtype=torch.float32, device=dev)
            gp = torch.zeros(N, dtype=torch.int16, device=dev)
            om, ov, omaster, oparam = (np.zeros(N, np.float32), np.zeros(N, np.float32), master0.copy(),
                                       np.zeros(N, np.uint16))
            ws = ws_tensor(torch, z.workspace_bytes(N, W), dev)
            gbuf = torch.empty(N, dtype=torch.float32, device=dev)
            for t in range(1, 4):
                G = replicas(77 + variant, t, W, N, [0.02, 0.3, 1e-4][t % 3])
                gd = [to_dev_u16(torch, x, dev) for x in G]
                g_o = oracle.shard_reduce(G)
                if variant & oracle.G_BF16:
                    g_o = oracle.round_to_bf16(g_o)
                mx = oracle.global_norm([oracle.sumsq(g_o)]) if t == 2 else 1.0
                rs = np.zeros(1)
                oi = oracle.step(G, omaster, om, ov, oparam, hp_at(t, max_norm=mx), rs, 0, variant=variant)
                if t == 2:
                    assert oi.clip == bool(variant & oracle.CLIP_EPS)
                rsd = torch.zeros(1, dtype=torch.float64, device=dev)
                info = torch.zeros(4, dtype=torch.float64, device=dev)
                z.shard_reduce(gd, 0, N, g_out=gbuf, sumsq_out=rsd, flags=fl, ws=ws)
                rsd.copy_(torch.from_numpy(rs))      # the oracle's partial, so that the norm is the same
                if recompute:
                    z.adamw_step(None, gd, 0, N, gm, gmm, gvv, gp, hp_at(t, max_norm=mx), rsd, 1, flags=fl,
                                 info_out=info)
                else:
                    z.adamw_step(gbuf, None, 0, N, gm, gmm, gvv, gp, hp_at(t, max_norm=mx), rsd, 1, flags=fl,
                                 info_out=info)
                torch.cuda.synchronize()
                ni = info.cpu().numpy()
                assert rel_close(ni[1], oi.norm, NORM_TOL)
                assert bool(ni[2:4].view(np.int32)[1]) == oi.clip and ni[2:3].view(np.float32)[0] == oi.coef
            what = f"flat variant={variant} recompute={recompute}"
            assert_f32_equal(gm.cpu().numpy(), omaster, "master " + what)
            assert_f32_equal(gmm.cpu().numpy(), om, "m " + what)
            assert_f32_equal(gvv.cpu().numpy(), ov, "v " + what)
            assert_bf16_equal(to_np_u16(gp), oparam, "param " + what)


def test_mta_misaligned_pieces(env):
    """Pieces whose lengths are not multiples of 8 make later pieces start off
    the 16-byte grid: the library must take its element-wise path and still
    match the oracle."""
    torch, dev = env
    run_mta_all_ranks(torch, dev, [13, 1001, 7, 4099, 65536 + 1], 3, 3, 0xC000, 0, False, False,
                      lambda t: 0.1)


@pytest.mark.parametrize("design", [0, z.STORE_G, z.RECOMPUTE_G])
def test_c1_full_trajectory(env, design):
    """The flat 2^20-parameter model at W=4, every rank, 10 steps, against the
    oracle (design 0: the library's choice, recompute at W = 4)."""
    from synth.workloads import configs
    c = configs()["C1"]
    torch, dev = env
    run_mta_all_ranks(torch, dev, [c.n_total], c.W, c.steps, c.seed, design, False, True,
                      lambda t: c.sigma)


# ---------------------------------------------------------------- properties
def test_mta_equals_reduce_plus_adamw(env):
    torch, dev = env
    W, numels = 8, [50000, 3, 70001]
    N = sum(numels)
    r = 5
    master_full = synth.f32(N, synth.master_key(9), 0, 0.02)
    a = MtaShard(torch, dev, numels, W, r, master_full)
    b0, S = a.begin, a.S
    fm = torch.from_numpy(master_full[b0:b0 + S].copy()).to(dev)
    fmm = torch.zeros(S, dtype=torch.float32, device=dev)
    fvv = torch.zeros(S, dtype=torch.float32, device=dev)
    fp = torch.zeros(S, dtype=torch.int16, device=dev)
    ws1, ws2 = a.workspace(z.STORE_G), ws_tensor(torch, z.workspace_bytes(S, W), dev)
    g = torch.empty(S, dtype=torch.float32, device=dev)
    for t in range(1, 4):
        G = replicas(9, t, W, N, 0.3)
        gd = [to_dev_u16(torch, x, dev) for x in G]
        rs1 = torch.full((W,), 0.125, dtype=torch.float64, device=dev)
        rs2 = rs1.clone()
        z.mta_step(gd, b0, a.plan, hp_at(t), rs1, W, r, flags=z.STORE_G, ws=ws1)
        z.shard_reduce(gd, b0, S, g_out=g, sumsq_out=rs2[r:r + 1], ws=ws2)
        z.adamw_step(g, None, 0, S, fm, fmm, fvv, fp, hp_at(t), rs2, W)
        torch.cuda.synchronize()
        assert rs1[r].item() == rs2[r].item()
    master, m, v, param = a.gather()
    assert_f32_equal(master, fm.cpu().numpy(), "master")
    assert_f32_equal(m, fmm.cpu().numpy(), "m")
    assert_f32_equal(v, fvv.cpu().numpy(), "v")
    assert_bf16_equal(param, to_np_u16(fp), "param")


def test_rerun_is_bit_identical_and_resume_is_exact(env):
    torch, dev = env
    W, numels, r = 4, [100_000, 33_333, 7], 2
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(11), 0, 0.02)
    runs = []
    for mode in ("straight", "straight", "resume"):
        a = MtaShard(torch, dev, numels, W, r, master_full)
        ws = a.workspace()
        norms = []
        for t in range(1, 7):
            if mode == "resume" and t == 4:
                # checkpoint m, v, master (t is an argument), then restore into fresh buffers
                saved = [tuple(x.clone().cpu() for x in s) for s in a.state]
                a = MtaShard(torch, dev, numels, W, r, master_full)
                ws = a.workspace()
                for dst, src in zip(a.state, saved):
                    for d, s in zip(dst, src):
                        d.copy_(s.to(dev))
            G = replicas(11, t, W, N, 0.2)
            gd = [to_dev_u16(torch, x, dev) for x in G]
            rs = torch.full((W,), 0.5, dtype=torch.float64, device=dev)
            info = torch.zeros(4, dtype=torch.float64, device=dev)
            z.mta_step(gd, a.begin, a.plan, hp_at(t), rs, W, r, info_out=info, ws=ws)
            torch.cuda.synchronize()
            norms.append(info.cpu().numpy().tobytes())
        runs.append((a.gather(), norms))
    (s0, n0), (s1, n1), (s2, n2) = runs
    assert n0 == n1 == n2
    for x, y, q in zip(s0, s1, s2):
        assert x.tobytes() == y.tobytes() == q.tobytes()


def test_nonfinite_gradient_propagates(env):
    torch, dev = env
    W, N = 3, 30000
    G = replicas(21, 1, W, N, 0.01)
    G[1][12345] = 0x7FC0          # NaN in one replica
    G[2][777] = 0x7F80            # +inf in another
    master0 = synth.f32(N, synth.master_key(21), 0, 0.02)
    for max_norm in (1.0, math.inf):
        om, ov = np.zeros(N, np.float32), np.zeros(N, np.float32)
        omaster, oparam = master0.copy(), np.zeros(N, np.uint16)
        rs = np.zeros(1)
        oi = oracle.step(G, omaster, om, ov, oparam, hp_at(1, max_norm=max_norm), rs, 0)
        gd = [to_dev_u16(torch, x, dev) for x in G]
        gm = torch.from_numpy(master0.copy()).to(dev)
        gmm = torch.zeros(N, dtype=torch.float32, device=dev)
        gvv = torch.zeros(N, dtype=torch.float32, device=dev)
        gp = torch.zeros(N, dtype=torch.int16, device=dev)
        ws = ws_tensor(torch, z.workspace_bytes(N, W), dev)
        rsd = torch.zeros(1, dtype=torch.float64, device=dev)
        info = torch.zeros(4, dtype=torch.float64, device=dev)
        z.shard_reduce(gd, 0, N, sumsq_out=rsd, ws=ws)
        z.adamw_step(None, gd, 0, N, gm, gmm, gvv, gp, hp_at(1, max_norm=max_norm), rsd, 1,
                     info_out=info)
        torch.cuda.synchronize()
        ni = info.cpu().numpy()
        assert np.isnan(ni[1]) and np.isnan(oi.norm)
        assert ni[2:4].view(np.int32)[1] == 0 and not oi.clip      # NaN norm: no clip
        assert info.cpu().numpy()[3:4].view(np.int32)[0] == 1       # nonfinite flag
        assert_f32_equal(gm.cpu().numpy(), omaster, "master with NaN/inf")
        assert_bf16_equal(to_np_u16(gp), oparam, "param with NaN/inf")


def test_bf16_stagnation_on_gpu(env):
    """A constant +2^-10 gradient, lr=1e-3, no decay, no clip, 1000 steps from
    master 1.0: the fp32 master walks to ~0 exactly as the oracle does, and the
    bf16 parameter follows it instead of sticking at 1.0."""
    torch, dev = env
    n = 64
    g = np.full(n, 0x3A80, dtype=np.uint16)          # 2^-10 in bf16
    gd = [to_dev_u16(torch, g, dev)]
    gm = torch.ones(n, dtype=torch.float32, device=dev)
    gmm = torch.zeros(n, dtype=torch.float32, device=dev)
    gvv = torch.zeros(n, dtype=torch.float32, device=dev)
    gp = torch.zeros(n, dtype=torch.int16, device=dev)
    ws = ws_tensor(torch, z.workspace_bytes(n, 1), dev)
    rsd = torch.zeros(1, dtype=torch.float64, device=dev)
    om, ov = np.zeros(n, np.float32), np.zeros(n, np.float32)
    omaster, oparam = np.ones(n, np.float32), np.zeros(n, np.uint16)
    for t in range(1, 1001):
        hp = hp_at(t, weight_decay=0.0, max_norm=math.inf)
        z.shard_reduce(gd, 0, n, sumsq_out=rsd, ws=ws)
        z.adamw_step(None, gd, 0, n, gm, gmm, gvv, gp, hp, rsd, 1)
        oracle.step([g], omaster, om, ov, oparam, hp, np.zeros(1), 0)
    torch.cuda.synchronize()
    assert_f32_equal(gm.cpu().numpy(), omaster, "master after 1000 steps")
    assert abs(float(omaster[0])) < 2e-3
    p = to_np_u16(gp)
    assert_bf16_equal(p, oparam, "param after 1000 steps")
    assert np.all(oracle.bf16_to_f32(p) < 2e-3)


def test_bucketed_reduction_matches_oracle_and_mta_step(env):
    """ZeRO-2-style flow: each tensor's piece of the shard is a bucket whose W
    gradient slices exist only while it is reduced (reduced in reverse order,
    as backward produces them); the bucket partials are then added in order and
    the update runs alone.  State must equal the oracle's step bit for bit."""
    torch, dev = env
    W, steps = 4, 3
    numels = RAGGED8
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xE000), 0, 0.02)
    for r in (0, 3):
        sh = MtaShard(torch, dev, numels, W, r, master_full)
        ws = sh.workspace(z.STORE_G)
        from tests.oracle_sim import RankState
        o = RankState(master_full[sh.begin:sh.begin + sh.S])
        parts = torch.zeros(len(sh.pl), dtype=torch.float64, device=dev)
        rsd = torch.zeros(W, dtype=torch.float64, device=dev)
        info = torch.zeros(4, dtype=torch.float64, device=dev)
        for t in range(1, steps + 1):
            G = replicas(0xE000, t, W, N, [0.02, 1e-4, 0.3][t % 3])
            part = np.zeros(W)
            for q in range(W):
                b, e = shard_range(N, W, q)
                part[q] = oracle.sumsq(oracle.shard_reduce([g[b:e] for g in G]))
            for k in reversed(range(len(sh.pl))):
                _, _, so, n = sh.pl[k]
                lo = sh.begin + so
                bucket = [to_dev_u16(torch, g[lo:lo + n].copy(), dev) for g in G]   # this bucket only
                z.mta_reduce_range(bucket, sh.plan, so, so + n, parts[k:k + 1], flags=z.STORE_G, ws=ws)
                del bucket
            rsd.copy_(torch.from_numpy(part))
            z.partials_sum(parts, len(sh.pl), rsd[r:r + 1])
            gd = [to_dev_u16(torch, g, dev) for g in G]
            z.mta_update(gd, sh.begin, sh.plan, hp_at(t), rsd, W, flags=z.STORE_G, info_out=info, ws=ws)
            torch.cuda.synchronize()
            rs = part.copy()
            oi = oracle.step([g[sh.begin:sh.begin + sh.S] for g in G], o.master, o.m, o.v, o.param, hp_at(t), rs, r)
            ni = info.cpu().numpy()
            assert rel_close(rsd[r].item(), part[r], NORM_TOL)
            assert rel_close(ni[1], oi.norm, NORM_TOL)
            assert bool(ni[2:4].view(np.int32)[1]) == oi.clip and ni[2:3].view(np.float32)[0] == oi.coef
        master, m, v, p = sh.gather()
        what = f"bucketed rank {r}"
        assert_f32_equal(master, o.master, "master " + what)
        assert_f32_equal(m, o.m, "m " + what)
        assert_f32_equal(v, o.v, "v " + what)
        assert_bf16_equal(p, o.param, "param " + what)
    with pytest.raises(z.Zero1Error):
        z.mta_reduce_range(gd, sh.plan, 5, 3, parts[:1], ws=ws)
    with pytest.raises(z.Zero1Error):
        z.mta_reduce_range(gd, sh.plan, 0, 10, parts[:1], flags=z.RECOMPUTE_G, ws=ws)


@pytest.mark.parametrize("W", [127, 128])
def test_shard_reduce_widest(env, W):
    """The widest replica count the library takes (128) and an odd one next to
    it (127: the IEEE-division average), over ragged lengths and a misaligned
    start; the 4-slice load batches run to their ragged last batch."""
    torch, dev = env
    ws = ws_tensor(torch, z.workspace_bytes(1 << 16, W), dev)
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    for length, offset in [(1, 0), (2049, 3), (3 * 2048 + 17, 0)]:
        N = offset + length + 5
        G = replicas(3000 + W, length, W, N, 0.5, outlier_pct=2, specials=2)
        gd = [to_dev_u16(torch, g, dev) for g in G]
        gout = torch.full((length + 4,), float("nan"), dtype=torch.float32, device=dev)
        z.shard_reduce(gd, offset, length, g_out=gout, sumsq_out=sumsq, ws=ws)
        torch.cuda.synchronize()
        exp = oracle.shard_reduce([g[offset:offset + length] for g in G])
        assert_f32_equal(gout[:length].cpu().numpy(), exp, f"g W={W} len={length} off={offset}")
        assert np.isnan(gout[length:].cpu().numpy()).all(), "wrote past the end"
        assert rel_close(float(sumsq.item()), oracle.sumsq(exp), NORM_TOL)


def test_mta_widest_replica_count(env):
    """A whole ragged step at W=128 for two ranks (the slice pointers of all
    128 replicas travel in the kernel argument)."""
    torch, dev = env
    numels = [3000, 1, 70000, 129, 4096]
    for design in (z.STORE_G, z.RECOMPUTE_G):
        run_mta_all_ranks(torch, dev, numels, 128, 2, 0xF100, design, False, True,
                          lambda t: [0.02, 0.3][t % 2], ranks=[0, 77])


def test_mta_many_tiny_tensors(env):
    """A tensor list of 1,500 mostly tiny tensors (1 to 40 elements, a few
    larger), so most pieces are shorter than a lane group and many shards cut
    through the middle of one; every rank, both streaming designs."""
    torch, dev = env
    rng = np.random.default_rng(0x71A1)
    numels = [int(x) for x in rng.integers(1, 41, size=1500)]
    for i in (10, 700, 1499):
        numels[i] = 5000 + i
    for design in (z.STORE_G, z.RECOMPUTE_G):
        run_mta_all_ranks(torch, dev, numels, 3, 2, 0xF200, design, False, True,
                          lambda t: [0.02, 0.3][t % 2])


@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_mta_step_in_planned_arena(env, design):
    """Every array of one rank placed in one allocation by zero1_arena_plan
    (the spaced arrays 40 GiB apart, full replica gradients packed after the
    parameter buffer): two steps, bit-exact against the oracle, and nothing
    outside the arrays is written."""
    torch, dev = env
    numels = [3000, 17, 5000, 65536 + 3, 8192 * 2 + 1]
    N, W, r = sum(numels), 4, 1
    begin, S = z.shard_range(N, W, r)
    L = z.arena_plan(S, W, N, begin, N, begin, flags=design)
    assert L.spacing >= 40 << 30
    arena = torch.empty(L.total_bytes, dtype=torch.uint8, device=dev)
    guard = 4096   # sentinel bytes after every array

    def view(off, n, dt):
        nb = n * torch.empty((), dtype=dt).element_size()
        arena[off + nb:off + nb + guard].fill_(0xA5)
        return arena[off:off + nb].view(dt)
    grads = [arena[L.grads[w]:L.grads[w] + 2 * N].view(torch.int16) for w in range(W)]
    master = view(L.master, S, torch.float32)
    m = view(L.m, S, torch.float32)
    v = view(L.v, S, torch.float32)
    params = arena[L.params:L.params + 2 * N].view(torch.int16)
    ws = (view if design == z.STORE_G else lambda o, n, d: arena[o:o + n].view(d))(L.ws, L.ws_bytes, torch.uint8)
    master_full = synth.f32(N, synth.master_key(0xF300), 0, 0.02)
    master.copy_(torch.from_numpy(master_full[begin:begin + S].copy()))
    m.zero_()
    v.zero_()
    params.zero_()
    from tests.oracle_sim import RankState
    o = RankState(master_full[begin:begin + S])
    offs = np.concatenate([[0], np.cumsum(numels)])
    pieces = [(n, so, params[offs[ti] + off:], master[so:], m[so:], v[so:])
              for ti, off, so, n in z.shard_pieces(numels, begin, begin + S)]
    table = torch.empty(max(256, z.mta_table_bytes(pieces)), dtype=torch.uint8, device=dev)
    plan = z.mta_plan(pieces, table)
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    for t in (1, 2):
        G = replicas(0xF300, t, W, N, [0.02, 0.3][t - 1], outlier_pct=1)
        for w in range(W):
            grads[w].copy_(torch.from_numpy(G[w].view(np.int16)))
        part = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                         for b, n in (z.shard_range(N, W, q) for q in range(W))])
        rsd.copy_(torch.from_numpy(part))
        z.mta_step(grads, begin, plan, hp_at(t), rsd, W, r, flags=design, ws=ws)
        torch.cuda.synchronize()
        oracle.step([g[begin:begin + S] for g in G], o.master, o.m, o.v, o.param, hp_at(t), part.copy(), r)
    assert_f32_equal(master.cpu().numpy(), o.master, "master in arena")
    assert_f32_equal(m.cpu().numpy(), o.m, "m in arena")
    assert_f32_equal(v.cpu().numpy(), o.v, "v in arena")
    assert_bf16_equal(to_np_u16(params[begin:begin + S]), o.param, "params in arena")
    # the parameters outside the shard and the guard bands after the spaced
    # arrays (each followed by a gap) are untouched
    p_all = to_np_u16(params)
    assert not p_all[:begin].any() and not p_all[begin + S:].any()
    spaced = [(L.master, 4 * S), (L.m, 4 * S), (L.v, 4 * S)] + ([(L.ws, L.ws_bytes)] if design == z.STORE_G else [])
    for off, nb in spaced:
        assert (arena[off + nb:off + nb + guard] == 0xA5).all(), "wrote past an array"
    del arena
    torch.cuda.empty_cache()


@pytest.mark.parametrize("W,mv_bf16", [(8, False), (3, True)])
def test_arena_tensors_step(env, W, mv_bf16):
    """The arena helper as a training loop would use it: z.arena_tensors for
    the rank's arrays (full replica gradients, the whole parameter buffer),
    the plan built over its views, two steps with the design the library
    picks (store-g at W = 8, recompute at W = 3): bit-exact against the
    oracle, and the parameters outside the shard untouched."""
    torch, dev = env
    numels = RAGGED
    N, r = sum(numels), 1
    begin, S = z.shard_range(N, W, r)
    flags = z.MV_BF16 if mv_bf16 else 0
    a = z.arena_tensors(S, W, N, begin, N, begin, flags=flags, device=dev)
    master_full = synth.f32(N, synth.master_key(0xF400 + W), 0, 0.02)
    a.master.copy_(torch.from_numpy(master_full[begin:begin + S].copy()))
    a.m.zero_()
    a.v.zero_()
    a.params.zero_()
    from tests.oracle_sim import RankState
    o = RankState(master_full[begin:begin + S], mv_bf16)
    offs = np.concatenate([[0], np.cumsum(numels)])
    pieces = [(n, so, a.params[offs[ti] + off:], a.master[so:], a.m[so:], a.v[so:])
              for ti, off, so, n in z.shard_pieces(numels, begin, begin + S)]
    table = torch.empty(max(256, z.mta_table_bytes(pieces)), dtype=torch.uint8, device=dev)
    plan = z.mta_plan(pieces, table, flags=flags)
    assert z.mta_design(a.grads, begin, plan) == (z.STORE_G if W > 4 else z.RECOMPUTE_G)
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    for t in (1, 2):
        G = replicas(0xF400 + W, t, W, N, [0.02, 0.3][t - 1], outlier_pct=1)
        for w in range(W):
            a.grads[w].copy_(torch.from_numpy(G[w].view(np.int16)))
        part = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                         for b, n in (z.shard_range(N, W, q) for q in range(W))])
        rsd.copy_(torch.from_numpy(part))
        z.mta_step(a.grads, begin, plan, hp_at(t), rsd, W, r, ws=a.ws)
        torch.cuda.synchronize()
        oracle.step([g[begin:begin + S] for g in G], o.master, o.m, o.v, o.param, hp_at(t), part.copy(), r)
    assert_f32_equal(a.master.cpu().numpy(), o.master, "master")
    if mv_bf16:
        assert_bf16_equal(to_np_u16(a.m), o.m, "m")
        assert_bf16_equal(to_np_u16(a.v), o.v, "v")
    else:
        assert_f32_equal(a.m.cpu().numpy(), o.m, "m")
        assert_f32_equal(a.v.cpu().numpy(), o.v, "v")
    p_all = to_np_u16(a.params)
    assert_bf16_equal(p_all[begin:begin + S], o.param, "params")
    assert not p_all[:begin].any() and not p_all[begin + S:].any()
    del a
    torch.cuda.empty_cache()


@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_mta_step_captured_in_a_graph(env, design):
    """The step captured into a HIP graph (torch.cuda.graph) and replayed three
    times, with eager work and synchronizations between the replays, gives
    bit for bit the state of three eager calls with the same arguments."""
    torch, dev = env
    numels, W, r = RAGGED, 4, 2
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF400), 0, 0.02)
    eager = MtaShard(torch, dev, numels, W, r, master_full)
    graphed = MtaShard(torch, dev, numels, W, r, master_full)
    ws_e, ws_g = eager.workspace(design), graphed.workspace(design)
    G = replicas(0xF400, 1, W, N, 0.3, outlier_pct=1)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    part = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                     for b, n in (z.shard_range(N, W, q) for q in range(W))])
    rsd_e = torch.from_numpy(part.copy()).to(dev)
    rsd_g = torch.from_numpy(part.copy()).to(dev)
    info_e = torch.zeros(4, dtype=torch.float64, device=dev)
    info_g = torch.zeros(4, dtype=torch.float64, device=dev)
    hp = hp_at(1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        z.mta_step(gd, eager.begin, graphed.plan, hp, rsd_g, W, r, flags=design, info_out=info_g, ws=ws_g)
    torch.cuda.synchronize()
    scratch = torch.ones(1 << 20, device=dev)
    for k in range(3):
        z.mta_step(gd, eager.begin, eager.plan, hp, rsd_e, W, r, flags=design, info_out=info_e, ws=ws_e)
        graph.replay()
        scratch.mul_(1.0001).add_(1.0)        # eager work between the replays
        torch.cuda.synchronize()
        a, b = eager.gather(), graphed.gather()
        what = f"replay {k} design {design}"
        assert_f32_equal(b[0], a[0], "master " + what)
        assert_f32_equal(b[1], a[1], "m " + what)
        assert_f32_equal(b[2], a[2], "v " + what)
        assert_bf16_equal(b[3], a[3], "param " + what)
        assert rsd_g[r].item() == rsd_e[r].item()
        assert torch.equal(info_g, info_e)
        assert graphed.untouched_outside()
    del graph


@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_device_scalars_replay_changes_step_and_lr(env, design):
    """One step captured with its hyper-parameters in device memory, replayed
    for t = 1..4 under a changing learning rate (the scalars of each step
    derived on the host and copied in before its replay), equals four eager
    calls with host hyper-parameters and the oracle's four steps."""
    torch, dev = env
    numels, W, r = RAGGED8, 4, 3
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF500), 0, 0.02)
    eager = MtaShard(torch, dev, numels, W, r, master_full)
    replay = MtaShard(torch, dev, numels, W, r, master_full)
    ws_e, ws_g = eager.workspace(design), replay.workspace(design)
    from tests.oracle_sim import RankState
    o = RankState(master_full[eager.begin:eager.begin + eager.S])
    G = replicas(0xF500, 1, W, N, 0.3, outlier_pct=1)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    part = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                     for b, n in (z.shard_range(N, W, q) for q in range(W))])
    rsd_e = torch.from_numpy(part.copy()).to(dev)
    rsd_g = torch.from_numpy(part.copy()).to(dev)
    dev_scal = torch.zeros(5, dtype=torch.float64, device=dev)          # 40 bytes, 8-aligned
    host_scal = torch.zeros(40, dtype=torch.uint8).pin_memory()
    hp_dev = {"device_scalars": dev_scal}
    step = lambda: z.mta_step(gd, replay.begin, replay.plan, hp_dev, rsd_g, W, r, flags=design, ws=ws_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for t, lr in [(1, 1e-3), (2, 6e-4), (3, 3e-4), (4, 1e-4)]:
        hp = hp_at(t, lr=lr)
        s = z.step_scalars_derive(hp)
        host_scal.copy_(torch.frombuffer(bytearray(bytes(s)), dtype=torch.uint8))
        dev_scal.view(torch.uint8).copy_(host_scal, non_blocking=True)
        graph.replay()
        z.mta_step(gd, eager.begin, eager.plan, hp, rsd_e, W, r, flags=design, ws=ws_e)
        torch.cuda.synchronize()
        oracle.step([g[eager.begin:eager.begin + eager.S] for g in G], o.master, o.m, o.v, o.param, hp,
                    part.copy(), r)
        a, b = eager.gather(), replay.gather()
        what = f"t={t} design {design}"
        for k, name in ((0, "master"), (1, "m"), (2, "v")):
            assert_f32_equal(b[k], a[k], name + " replay vs eager " + what)
        assert_bf16_equal(b[3], a[3], "param replay vs eager " + what)
    master, m, v, p = replay.gather()
    assert_f32_equal(master, o.master, "master vs oracle")
    assert_f32_equal(m, o.m, "m vs oracle")
    assert_f32_equal(v, o.v, "v vs oracle")
    assert_bf16_equal(p, o.param, "param vs oracle")
    del graph


def test_workspace_errors(env):
    """A missing, misaligned or short workspace is rejected (EWORKSPACE) before
    anything is launched, on every entry point that takes one."""
    torch, dev = env
    numels, W, r = RAGGED, 4, 1
    N = sum(numels)
    sh = MtaShard(torch, dev, numels, W, r, synth.f32(N, synth.master_key(0xF600), 0, 0.02))
    G = replicas(0xF600, 1, W, N, 0.02)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    need_mta = z.mta_workspace_bytes(sh.plan, W, z.STORE_G)
    need_sr = z.workspace_bytes(5000, W)
    big = torch.empty(need_mta + need_sr + 512, dtype=torch.uint8, device=dev)
    base = big.data_ptr()
    calls = {
        "mta_step": (need_mta, lambda ws, nb: z.mta_step(gd, sh.begin, sh.plan, hp_at(1), rsd, W, r,
                                                         flags=z.STORE_G, ws=ws, ws_bytes=nb)),
        "mta_reduce": (need_mta, lambda ws, nb: z.mta_reduce(gd, sh.begin, sh.plan, rsd[r:r + 1],
                                                             flags=z.STORE_G, ws=ws, ws_bytes=nb)),
        "shard_reduce": (need_sr, lambda ws, nb: z.shard_reduce(gd, 0, 5000, sumsq_out=rsd[0:1], ws=ws,
                                                                ws_bytes=nb)),
    }
    for name, (need, call) in calls.items():
        for ws, nb, msg in [(None, None, "NULL"), (base + 16, need, "aligned"), (base, need - 1, "needs")]:
            with pytest.raises(z.Zero1Error) as e:
                call(ws, nb)
            assert e.value.name == "ZERO1_EWORKSPACE", (name, e.value)
            assert msg in e.value.message, (name, e.value.message)
    torch.cuda.synchronize()
    master, m, v, p = sh.gather()
    assert not m.any() and not v.any(), "a rejected call changed the state"


def test_c_program_runs_the_step(env, tmp_path):
    """tests/c/step_demo.c -- plain C11 over the HIP runtime and libzero1.so,
    no Python or torch -- runs three steps of a ragged tensor list for one
    rank; its master, m, v, bf16 params and norm info equal the oracle's."""
    import shutil
    import subprocess
    import os
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(z.lib_path)
    exe = tmp_path / "step_demo"
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
                    "-isystem", "/opt/rocm/include", "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c", "step_demo.c"), "-o", str(exe), "-L", libdir, "-lzero1",
                    "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True)
    sizes, W, r, steps = RAGGED, 4, 2, 3
    N = sum(sizes)
    b, S = z.shard_range(N, W, r)
    master_full = synth.f32(N, synth.master_key(0xF700), 0, 0.02)
    Gs = [replicas(0xF700, t, W, N, [0.3, 1e-4, 0.02][t - 1], outlier_pct=1) for t in range(1, steps + 1)]
    parts = np.array([[oracle.sumsq(oracle.shard_reduce([g[q0:q0 + n] for g in G]))
                       for q0, n in (z.shard_range(N, W, q) for q in range(W))] for G in Gs])
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([len(sizes), W, r, steps], dtype=np.int64).tobytes())
        f.write(np.array(sizes, dtype=np.int64).tobytes())
        f.write(parts.astype(np.float64).tobytes())
        f.write(master_full[b:b + S].astype(np.float32).tobytes())
        for G in Gs:
            for g in G:
                f.write(g.astype(np.uint16).tobytes())
    res = subprocess.run([str(exe), str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = np.fromfile(outp, dtype=np.uint8)
    master = raw[:4 * S].view(np.float32)
    m = raw[4 * S:8 * S].view(np.float32)
    v = raw[8 * S:12 * S].view(np.float32)
    param = raw[12 * S:14 * S].view(np.uint16)
    infos = raw[14 * S:].view(np.float64).reshape(steps, 4)
    from tests.oracle_sim import RankState
    o = RankState(master_full[b:b + S])
    for t, G in enumerate(Gs, start=1):
        oi = oracle.step([g[b:b + S] for g in G], o.master, o.m, o.v, o.param, hp_at(t), parts[t - 1].copy(), r)
        ni = infos[t - 1]
        assert rel_close(ni[1], oi.norm, NORM_TOL)
        assert bool(ni[2:4].view(np.int32)[1]) == oi.clip and ni[2:3].view(np.float32)[0] == oi.coef
    assert_f32_equal(master, o.master, "master from the C program")
    assert_f32_equal(m, o.m, "m from the C program")
    assert_f32_equal(v, o.v, "v from the C program")
    assert_bf16_equal(param, o.param, "params from the C program")


def test_two_streams_run_two_ranks_concurrently(env):
    """Two ranks' steps enqueued on two streams (default priority) at the same
    time, each with its own workspace: both equal the oracle (the library keeps
    no per-call state outside the caller's buffers)."""
    torch, dev = env
    numels, W, steps = RAGGED, 4, 3
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF800), 0, 0.02)
    ranks = (0, 3)
    shards = {r: MtaShard(torch, dev, numels, W, r, master_full) for r in ranks}
    wss = {r: shards[r].workspace(z.STORE_G) for r in ranks}
    rsds = {r: torch.zeros(W, dtype=torch.float64, device=dev) for r in ranks}
    streams = {r: torch.cuda.Stream() for r in ranks}
    from tests.oracle_sim import RankState
    ost = {r: RankState(master_full[shards[r].begin:shards[r].begin + shards[r].S]) for r in ranks}
    for t in range(1, steps + 1):
        G = replicas(0xF800, t, W, N, [0.3, 0.02, 1e-4][t - 1], outlier_pct=1)
        gd = [to_dev_u16(torch, g, dev) for g in G]
        part = np.array([oracle.sumsq(oracle.shard_reduce([g[q0:q0 + n] for g in G]))
                         for q0, n in (z.shard_range(N, W, q) for q in range(W))])
        for r in ranks:
            rsds[r].copy_(torch.from_numpy(part))
        torch.cuda.synchronize()
        for r in ranks:
            with torch.cuda.stream(streams[r]):
                z.mta_step(gd, shards[r].begin, shards[r].plan, hp_at(t), rsds[r], W, r, flags=z.STORE_G,
                           ws=wss[r], stream=streams[r])
        torch.cuda.synchronize()
        for r in ranks:
            b, S = shards[r].begin, shards[r].S
            oracle.step([g[b:b + S] for g in G], ost[r].master, ost[r].m, ost[r].v, ost[r].param, hp_at(t),
                        part.copy(), r)
    for r in ranks:
        master, m, v, p = shards[r].gather()
        assert_f32_equal(master, ost[r].master, f"master rank {r}")
        assert_f32_equal(m, ost[r].m, f"m rank {r}")
        assert_f32_equal(v, ost[r].v, f"v rank {r}")
        assert_bf16_equal(p, ost[r].param, f"param rank {r}")


@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_zero_gradients(env, design):
    """Degenerate input: every replica's gradient is +0 (step 1) or -0 (step 2),
    then eps = 0 (step 3, 0/0 by IEEE).  Norm 0, no clip, a pure decay of the
    master, then NaN everywhere in step 3: all as the oracle."""
    torch, dev = env
    numels, W, r = RAGGED8, 4, 1
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF900), 0, 0.02)
    sh = MtaShard(torch, dev, numels, W, r, master_full)
    ws = sh.workspace(design)
    from tests.oracle_sim import RankState
    o = RankState(master_full[sh.begin:sh.begin + sh.S])
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    for t, bits, eps in [(1, 0x0000, 1e-8), (2, 0x8000, 1e-8), (3, 0x0000, 0.0)]:
        G = [np.full(N, bits, np.uint16) for _ in range(W)]
        gd = [to_dev_u16(torch, g, dev) for g in G]
        hp = hp_at(t, eps=eps)
        rsd.zero_()
        z.mta_step(gd, sh.begin, sh.plan, hp, rsd, W, r, flags=design, info_out=info, ws=ws)
        torch.cuda.synchronize()
        oi = oracle.step([g[sh.begin:sh.begin + sh.S] for g in G], o.master, o.m, o.v, o.param, hp, np.zeros(W), r)
        ni = info.cpu().numpy()
        assert ni[1] == 0.0 and oi.norm == 0.0
        assert not ni[2:4].view(np.int32)[1] and ni[2:3].view(np.float32)[0] == np.float32(1.0)
        master, m, v, p = sh.gather()
        what = f"t={t} design {design}"
        assert_f32_equal(master, o.master, "master " + what)
        assert_f32_equal(m, o.m, "m " + what)
        assert_f32_equal(v, o.v, "v " + what)
        assert_bf16_equal(p, o.param, "param " + what)
    assert np.isnan(master).all()


@pytest.mark.parametrize("case", range(20))
def test_random_configurations(env, case):
    """Seeded random configurations: replica count, tensor list (tiny, medium
    and large tensors mixed), rank, design, moment storage, state layout,
    compatibility variant and clip threshold, two steps each, bit-exact
    against the oracle."""
    torch, dev = env
    rng = np.random.default_rng(0xC0FFEE + case)
    W = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    aligned = case % 5 == 4
    n_t = int(rng.integers(1, 31))
    kinds = rng.choice(3, size=n_t, p=[0.4, 0.4, 0.2])
    sizes = [int(rng.integers(1, 41)) if k == 0 else int(rng.integers(100, 5001)) if k == 1
             else int(rng.integers(10000, 70001)) for k in kinds]
    if aligned:   # pieces and shard boundaries on 8-element boundaries (the vector path)
        sizes = [8 * max(1, s // 8) for s in sizes]
        S0 = -(-sum(sizes) // W)
        S0 = -(-S0 // 8) * 8
        sizes[-1] += W * S0 - sum(sizes)
    design = int(rng.choice([z.STORE_G, z.RECOMPUTE_G]))
    mv_bf16 = bool(rng.integers(0, 2))
    flat_state = bool(rng.integers(0, 2))
    variant = int(rng.choice([0, 0, oracle.DECAY_FIRST, oracle.CLIP_EPS, oracle.G_BF16,
                              oracle.DECAY_FIRST | oracle.CLIP_EPS]))
    max_norm = float(rng.choice([1.0, 0.05, math.inf]))
    scale = float(rng.choice([1e-4, 1e-2, 0.3]))
    r = int(rng.integers(0, W))
    _, S = z.shard_range(sum(sizes), W, r)
    if S == 0:
        r = 0
    run_mta_all_ranks(torch, dev, sizes, W, 2, 0xE100 + case, design, mv_bf16, flat_state,
                      lambda t: scale * (1 + t), max_norm=max_norm, ranks=[r], variant=variant)


@pytest.mark.parametrize("case", range(60))
def test_random_configurations_wide(env, case):
    """Seeded random configurations over the whole replica range (W up to
    128) with larger tensors (up to 300,000 elements each, any alignment):
    design, moment storage, state layout, compatibility variant and clip
    threshold drawn at random, two steps, one random rank, bit-exact against
    the oracle."""
    torch, dev = env
    rng = np.random.default_rng(0xF022 + case)
    W = int(rng.integers(1, 129))
    sizes = [int(rng.integers(1, 300001)) for _ in range(int(rng.integers(1, 12)))]
    design = int(rng.choice([z.STORE_G, z.RECOMPUTE_G]))
    mv_bf16 = bool(rng.integers(0, 2))
    flat_state = bool(rng.integers(0, 2))
    variant = int(rng.choice([0, 0, oracle.DECAY_FIRST, oracle.CLIP_EPS, oracle.G_BF16]))
    max_norm = float(rng.choice([1.0, 0.05, math.inf]))
    scale = float(rng.choice([1e-4, 1e-2, 0.3]))
    r = int(rng.integers(0, W))
    _, S = z.shard_range(sum(sizes), W, r)
    if S == 0:
        r = 0
    run_mta_all_ranks(torch, dev, sizes, W, 2, 0xF100 + case, design, mv_bf16, flat_state,
                      lambda t: scale * (1 + t), max_norm=max_norm, ranks=[r], variant=variant)


# (sum only, compatibility variant) of each random-cut case
BUCKET_VARIANTS = [(False, 0), (False, oracle.G_BF16 | oracle.DECAY_FIRST), (True, 0),
                   (True, oracle.CLIP_EPS | oracle.G_BF16)]


@pytest.mark.parametrize("case", range(4))
def test_bucketed_reduction_random_cuts(env, case):
    """Buckets cut at random points of the shard (most not on 8-element or
    tile boundaries, so both the vector and the element paths run), reduced
    in a random order, with the sum kept or averaged and with compatibility
    variants: the state equals the oracle's step."""
    torch, dev = env
    sum_only, variant = BUCKET_VARIANTS[case]
    flags = z.STORE_G | (z.SUM_ONLY if sum_only else 0) | lib_flags(variant)
    rflags = flags & (z.STORE_G | z.SUM_ONLY | z.G_BF16)    # what the bucket reduce takes
    rng = np.random.default_rng(0xB0C4 + case)
    W = int(rng.choice([2, 4, 8]))
    numels = RAGGED
    N = sum(numels)
    r = int(rng.integers(0, W))
    master_full = synth.f32(N, synth.master_key(0xE200 + case), 0, 0.02)
    sh = MtaShard(torch, dev, numels, W, r, master_full)
    ws = sh.workspace(z.STORE_G)
    from tests.oracle_sim import RankState
    o = RankState(master_full[sh.begin:sh.begin + sh.S])
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    for t in (1, 2):
        cuts = np.unique(np.concatenate([[0, sh.S], rng.integers(1, sh.S, size=int(rng.integers(1, 12)))]))
        ranges = list(zip(cuts[:-1], cuts[1:]))
        parts = torch.zeros(len(ranges), dtype=torch.float64, device=dev)
        G = replicas(0xE200 + case, t, W, N, 0.3, outlier_pct=1)
        def reduced(q0, n):
            gr = oracle.shard_reduce([g[q0:q0 + n] for g in G], average=not sum_only)
            return oracle.round_to_bf16(gr) if variant & oracle.G_BF16 else gr

        part = np.array([oracle.sumsq(reduced(q0, n)) for q0, n in (z.shard_range(N, W, q) for q in range(W))])
        for k in rng.permutation(len(ranges)):
            lo, hi = (int(x) for x in ranges[k])
            bucket = [to_dev_u16(torch, g[sh.begin + lo:sh.begin + hi].copy(), dev) for g in G]
            z.mta_reduce_range(bucket, sh.plan, lo, hi, parts[k:k + 1], flags=rflags, ws=ws)
        rsd.copy_(torch.from_numpy(part))
        z.partials_sum(parts, len(ranges), rsd[r:r + 1])
        gd = [to_dev_u16(torch, g, dev) for g in G]
        z.mta_update(gd, sh.begin, sh.plan, hp_at(t), rsd, W, flags=flags, ws=ws)
        torch.cuda.synchronize()
        assert rel_close(rsd[r].item(), part[r], NORM_TOL)
        oracle.step([g[sh.begin:sh.begin + sh.S] for g in G], o.master, o.m, o.v, o.param, hp_at(t), part.copy(), r,
                    average=not sum_only, variant=variant)
    master, m, v, p = sh.gather()
    assert_f32_equal(master, o.master, "master")
    assert_f32_equal(m, o.m, "m")
    assert_f32_equal(v, o.v, "v")
    assert_bf16_equal(p, o.param, "param")


@pytest.mark.parametrize("case", range(16))
def test_bucketed_reduction_random_wide(env, case):
    """The bucketed flow over random tensor lists and replica counts (W from 1
    to 128), up to 40 buckets cut anywhere and reduced in a random order, sum
    or average, fp32 or bf16 moments, flat or per-tensor state, compatibility
    variants, two steps.  The bucket partials' sum matches the oracle's
    partial to 1e-12; the update then gets the oracle's partials (so that the
    norm is the same double) and the state equals the oracle's bit for bit."""
    torch, dev = env
    rng = np.random.default_rng(0xB1D0 + case)
    W = int(rng.integers(1, 129))
    numels = [int(rng.integers(1, 100001)) for _ in range(int(rng.integers(1, 12)))]
    N = sum(numels)
    sum_only = bool(rng.integers(0, 4) == 0)
    variant = int(rng.choice([0, 0, oracle.DECAY_FIRST, oracle.CLIP_EPS, oracle.G_BF16]))
    mv_bf16 = bool(rng.integers(0, 2))
    flat_state = bool(rng.integers(0, 2))
    flags = z.STORE_G | (z.SUM_ONLY if sum_only else 0) | lib_flags(variant)
    rflags = flags & (z.STORE_G | z.SUM_ONLY | z.G_BF16)
    r = int(rng.integers(0, W))
    if z.shard_range(N, W, r)[1] == 0:
        r = 0
    seed = 0xE300 + case
    master_full = synth.f32(N, synth.master_key(seed), 0, 0.02)
    sh = MtaShard(torch, dev, numels, W, r, master_full, mv_bf16, flat_state)
    ws = sh.workspace(z.STORE_G)
    from tests.oracle_sim import RankState
    o = RankState(master_full[sh.begin:sh.begin + sh.S], mv_bf16)
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    what = f"case={case} W={W} numels={numels} rank={r} sum_only={sum_only} variant={variant} bf16mv={mv_bf16}"
    for t in (1, 2):
        n_cuts = int(rng.integers(0, 40))
        cuts = np.unique(np.concatenate([[0, sh.S], rng.integers(0, sh.S + 1, size=n_cuts)]))
        ranges = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:])]
        parts = torch.zeros(max(len(ranges), 1), dtype=torch.float64, device=dev)
        G = replicas(seed, t, W, N, float(rng.choice([1e-3, 0.3])), outlier_pct=1)

        def reduced(q0, n):
            gr = oracle.shard_reduce([g[q0:q0 + n] for g in G], average=not sum_only)
            return oracle.round_to_bf16(gr) if variant & oracle.G_BF16 else gr

        part = np.array([oracle.sumsq(reduced(q0, n)) for q0, n in (z.shard_range(N, W, q) for q in range(W))])
        for k in rng.permutation(len(ranges)):
            lo, hi = ranges[k]
            bucket = [to_dev_u16(torch, g[sh.begin + lo:sh.begin + hi].copy(), dev) for g in G]
            z.mta_reduce_range(bucket, sh.plan, lo, hi, parts[k:k + 1], flags=rflags, ws=ws)
        z.partials_sum(parts, len(ranges), rsd[r:r + 1])
        torch.cuda.synchronize()
        assert rel_close(rsd[r].item(), part[r], NORM_TOL), (what, rsd[r].item(), part[r])
        rsd.copy_(torch.from_numpy(part))
        gd = [to_dev_u16(torch, g, dev) for g in G]
        z.mta_update(gd, sh.begin, sh.plan, hp_at(t), rsd, W, flags=flags, ws=ws)
        torch.cuda.synchronize()
        oracle.step([g[sh.begin:sh.begin + sh.S] for g in G], o.master, o.m, o.v, o.param, hp_at(t), part.copy(), r,
                    average=not sum_only, variant=variant)
    master, m, v, p = sh.gather()
    assert_f32_equal(master, o.master, "master " + what)
    if mv_bf16:
        assert_bf16_equal(m, o.m, "m " + what)
        assert_bf16_equal(v, o.v, "v " + what)
    else:
        assert_f32_equal(m, o.m, "m " + what)
        assert_f32_equal(v, o.v, "v " + what)
    assert_bf16_equal(p, o.param, "param " + what)


def test_kernel_scoped_timing(env):
    """zero1_time_next_launch: a timed step gives bit for bit the state of an
    untimed one; each kernel's own duration is positive and the two together
    take less than the same calls bracketed by stream markers; a request is
    dropped when the next step call returns, also when that call fails; a
    capturing stream refuses it."""
    torch, dev = env
    numels, W, r = RAGGED8, 4, 1
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF600), 0, 0.02)
    timed = MtaShard(torch, dev, numels, W, r, master_full)
    plain = MtaShard(torch, dev, numels, W, r, master_full)
    ws_t, ws_p = timed.workspace(z.STORE_G), plain.workspace(z.STORE_G)
    G = replicas(0xF600, 1, W, N, 0.3, outlier_pct=1)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    part = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                     for b, n in (z.shard_range(N, W, q) for q in range(W))])
    rsd_t = torch.from_numpy(part.copy()).to(dev)
    rsd_p = torch.from_numpy(part.copy()).to(dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()          # torch creates the event at its first record
        return e

    for t in (1, 2, 3):
        hp = hp_at(t)
        rs, re_, us, ue, m0, m1 = (ev() for _ in range(6))
        m0.record()
        z.time_next_launch(rs, re_)
        z.mta_reduce(gd, timed.begin, timed.plan, rsd_t[r:r + 1], flags=z.STORE_G, ws=ws_t)
        z.time_next_launch(us, ue)
        z.mta_update(gd, timed.begin, timed.plan, hp, rsd_t, W, flags=z.STORE_G, ws=ws_t)
        m1.record()
        z.mta_step(gd, plain.begin, plain.plan, hp, rsd_p, W, r, flags=z.STORE_G, ws=ws_p)
        torch.cuda.synchronize()
        red, upd, whole = rs.elapsed_time(re_), us.elapsed_time(ue), m0.elapsed_time(m1)
        assert 0 < red and 0 < upd and red + upd < whole, (red, upd, whole)
        a, b = plain.gather(), timed.gather()
        for k, name in ((0, "master"), (1, "m"), (2, "v")):
            assert_f32_equal(b[k], a[k], f"{name} timed vs untimed t={t}")
        assert_bf16_equal(b[3], a[3], f"param timed vs untimed t={t}")
        assert rsd_t[r].item() == rsd_p[r].item()

    # dropped when the next step call returns, even a failing one: the later
    # untimed reduce leaves the two creation stamps as they were
    a, b = ev(), ev()
    torch.cuda.synchronize()
    before = a.elapsed_time(b)
    z.time_next_launch(a, b)
    with pytest.raises(z.Zero1Error) as ei:
        z.mta_reduce(gd, timed.begin, timed.plan, None, flags=z.STORE_G, ws=ws_t)
    assert ei.value.name == "ZERO1_EINVAL"
    z.mta_reduce(gd, timed.begin, timed.plan, rsd_t[r:r + 1], flags=z.STORE_G, ws=ws_t)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == before

    # a stream being captured refuses the request before launching; the same
    # call without it is captured and replays like an eager call
    q_graph = torch.zeros(1, dtype=torch.float64, device=dev)
    q_eager = torch.zeros(1, dtype=torch.float64, device=dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(graph):
        z.time_next_launch(a, b)
        try:
            z.mta_reduce(gd, timed.begin, timed.plan, q_graph, flags=z.STORE_G, ws=ws_t)
        except z.Zero1Error as e:
            refused = e
        z.mta_reduce(gd, timed.begin, timed.plan, q_graph, flags=z.STORE_G, ws=ws_t)
    assert refused is not None and refused.name == "ZERO1_EHIP", refused
    graph.replay()
    z.mta_reduce(gd, timed.begin, timed.plan, q_eager, flags=z.STORE_G, ws=ws_p)
    torch.cuda.synchronize()
    assert q_graph.item() == q_eager.item() == rsd_p[r].item()
    del graph


@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
@pytest.mark.parametrize("fault", ["nan_partial", "bit_flip", "inf_grad"])
def test_failure_injection(env, design, fault):
    """Faults forced from the host; the GPU step and the oracle agree on each:
    another rank's partial missing (NaN in its rank_sumsq entry) gives a NaN
    norm, no clip and the nonfinite flag; a flipped exponent bit in one
    replica's slice gives the same (wrong) step on both sides, which nothing
    in the step can detect; +inf in one gradient gives an infinite norm, a
    coefficient of 0 and NaN at that element only."""
    torch, dev = env
    from tests.oracle_sim import RankState
    numels, W, r = RAGGED8, 4, 1
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF700), 0, 0.02)
    sh = MtaShard(torch, dev, numels, W, r, master_full)
    ws = sh.workspace(design)
    o = RankState(master_full[sh.begin:sh.begin + sh.S])
    G = replicas(0xF700, 1, W, N, 0.3, outlier_pct=1)
    k = sh.begin + 1234                      # an element of this rank's shard
    if fault == "bit_flip":
        G[2][k] ^= 0x4000                    # the exponent's top bit
    elif fault == "inf_grad":
        G[0][k] = 0x7F80                     # +inf
    part = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                     for b, n in (z.shard_range(N, W, q) for q in range(W))])
    if fault == "nan_partial":
        part[3] = np.nan                     # rank 3's partial never arrived
    gd = [to_dev_u16(torch, g, dev) for g in G]
    rsd = torch.from_numpy(part.copy()).to(dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    z.mta_step(gd, sh.begin, sh.plan, hp_at(1), rsd, W, r, flags=design, info_out=info, ws=ws)
    orank = part.copy()
    oi = oracle.step([g[sh.begin:sh.begin + sh.S] for g in G], o.master, o.m, o.v, o.param, hp_at(1), orank, r)
    torch.cuda.synchronize()
    what = f"{fault} design {design}"
    master, m, v, p = sh.gather()
    assert_f32_equal(master, o.master, "master " + what)
    assert_f32_equal(m, o.m, "m " + what)
    assert_f32_equal(v, o.v, "v " + what)
    assert_bf16_equal(p, o.param, "param " + what)
    assert sh.untouched_outside()
    ni = info.cpu().numpy()
    iw = ni.view(np.int32)
    assert rel_close(ni[1], oi.norm, NORM_TOL) and rel_close(rsd[r].item(), orank[r], NORM_TOL)
    assert bool(iw[5]) == oi.clip and ni[2:3].view(np.float32)[0] == np.float32(oi.coef)
    assert iw[6] == int(not math.isfinite(oi.norm))
    if fault == "inf_grad":
        assert math.isinf(oi.norm) and oi.clip and oi.coef == 0.0
        j = k - sh.begin
        assert np.isnan(master[j]) and np.isnan(o.master).sum() == 1
    elif fault == "nan_partial":
        assert math.isnan(oi.norm) and not oi.clip
    else:
        assert math.isfinite(oi.norm) and oi.norm > 1e30 and oi.clip   # 0.3-ish value -> ~1e38


@pytest.mark.parametrize("design", [z.STORE_G, z.RECOMPUTE_G])
def test_zero1_equals_ddp_on_gpu(env, design):
    """ZeRO-1 is DDP with the optimizer state sharded: W ranks each reducing
    their slice, exchanging one partial each and updating their shard give,
    concatenated, bit for bit the state of one non-sharded step on the whole
    averaged gradient (norm from a single partial), over three steps."""
    torch, dev = env
    numels, W = RAGGED8, 4
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xF800), 0, 0.02)
    ranks = [MtaShard(torch, dev, numels, W, q, master_full) for q in range(W)]
    whole = MtaShard(torch, dev, numels, 1, 0, master_full)
    ws = [sh.workspace(design) for sh in ranks]
    ws_whole = whole.workspace(design)
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    q_whole = torch.zeros(1, dtype=torch.float64, device=dev)
    info_r = torch.zeros(4, dtype=torch.float64, device=dev)
    info_w = torch.zeros(4, dtype=torch.float64, device=dev)
    for t in (1, 2, 3):
        G = replicas(0xF800, t, W, N, 0.3 if t != 2 else 0.001, outlier_pct=1)   # clip, no clip, clip
        gd = [to_dev_u16(torch, g, dev) for g in G]
        hp = hp_at(t)
        for q, sh in enumerate(ranks):       # every rank's reduce, then the exchange of partials
            z.mta_reduce(gd, sh.begin, sh.plan, rsd[q:q + 1], flags=design, ws=ws[q])
        for q, sh in enumerate(ranks):
            z.mta_update(gd, sh.begin, sh.plan, hp, rsd, W, flags=design, info_out=info_r, ws=ws[q])
        z.mta_step(gd, 0, whole.plan, hp, q_whole, 1, 0, flags=design, info_out=info_w, ws=ws_whole)
        torch.cuda.synchronize()
        ni_r, ni_w = info_r.cpu().numpy(), info_w.cpu().numpy()
        assert rel_close(ni_r[1], ni_w[1], NORM_TOL)
        assert ni_r[2:3].view(np.float32)[0] == ni_w[2:3].view(np.float32)[0], "clip coefficients differ"
        parts = [sh.gather() for sh in ranks]
        ref = whole.gather()
        what = f"t={t} design {design}"
        for k, name in ((0, "master"), (1, "m"), (2, "v")):
            assert_f32_equal(np.concatenate([p[k] for p in parts]), ref[k], f"{name} ZeRO-1 vs DDP {what}")
        assert_bf16_equal(np.concatenate([p[3] for p in parts]), ref[3], f"param ZeRO-1 vs DDP {what}")


def test_clip_threshold_is_strict(env):
    """Gradients of ±0.5 make every square and every partial sum exact, so the
    norm is exactly 256 on both sides whatever the summation order: a norm
    equal to max_norm is not clipped, one ulp of max_norm below it is (with
    the coefficient rounding to 1.0f), and max_norm = 128 halves g; the state
    matches the oracle each time."""
    torch, dev = env
    W, N = 2, 262144                        # 262144 * 0.25 = 65536 = 256^2
    sign = np.where(synth.bf16(N, synth.grad_key(0xF900, 1, 0), 0, 1.0) & 0x8000, 0xBF00, 0x3F00).astype(np.uint16)
    G = [sign.copy(), sign.copy()]          # both replicas ±0.5: g = ±0.5
    master0 = synth.f32(N, synth.master_key(0xF900), 0, 0.02)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    ws = ws_tensor(torch, z.workspace_bytes(N, W, z.STORE_G), dev)
    g = torch.empty(N, dtype=torch.float32, device=dev)
    for max_norm, clip, coef in [(256.0, False, 1.0), (math.nextafter(256.0, 0.0), True, 1.0),
                                 (128.0, True, 0.5), (math.nextafter(256.0, math.inf), False, 1.0)]:
        q = torch.zeros(1, dtype=torch.float64, device=dev)
        z.shard_reduce(gd, 0, N, g_out=g, sumsq_out=q, ws=ws)
        gm = torch.from_numpy(master0.copy()).to(dev)
        gmm = torch.zeros(N, dtype=torch.float32, device=dev)
        gvv = torch.zeros(N, dtype=torch.float32, device=dev)
        gp = torch.zeros(N, dtype=torch.int16, device=dev)
        info = torch.zeros(4, dtype=torch.float64, device=dev)
        hp = hp_at(1, max_norm=max_norm)
        z.adamw_step(g, None, 0, N, gm, gmm, gvv, gp, hp, q, 1, info_out=info)
        om, ov = np.zeros(N, np.float32), np.zeros(N, np.float32)
        omaster, oparam = master0.copy(), np.zeros(N, np.uint16)
        oi = oracle.step(G, omaster, om, ov, oparam, hp, np.zeros(1), 0)
        torch.cuda.synchronize()
        ni = info.cpu().numpy()
        assert q.item() == 65536.0 and ni[1] == 256.0 and oi.norm == 256.0
        assert bool(ni.view(np.int32)[5]) == clip == oi.clip, max_norm
        assert ni[2:3].view(np.float32)[0] == np.float32(coef) == np.float32(oi.coef), max_norm
        what = f"max_norm={max_norm!r}"
        assert_f32_equal(gm.cpu().numpy(), omaster, "master " + what)
        assert_f32_equal(gmm.cpu().numpy(), om, "m " + what)
        assert_f32_equal(gvv.cpu().numpy(), ov, "v " + what)
        assert_bf16_equal(to_np_u16(gp), oparam, "param " + what)


def test_host_threads_step_ranks_concurrently(env):
    """Four host threads, one rank each, step their ranks at the same time on
    their own streams (the binding releases the interpreter lock during each
    call), interleaved with rejected calls whose messages each thread reads
    back: every rank equals the oracle, and every thread sees its own error
    message (the library's error state is per thread)."""
    import threading
    torch, dev = env
    from tests.oracle_sim import RankState
    numels, W, steps = RAGGED8, 4, 3
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0xFA00), 0, 0.02)
    ranks = (0, 1, 2, 3)
    shards = {r: MtaShard(torch, dev, numels, W, r, master_full) for r in ranks}
    wss = {r: shards[r].workspace(z.STORE_G) for r in ranks}
    rsds = {r: torch.zeros(W, dtype=torch.float64, device=dev) for r in ranks}
    Gs, gds, parts = [], [], []
    for t in range(1, steps + 1):
        G = replicas(0xFA00, t, W, N, [0.3, 0.02, 1e-4][t - 1], outlier_pct=1)
        Gs.append(G)
        gds.append([to_dev_u16(torch, g, dev) for g in G])
        parts.append(np.array([oracle.sumsq(oracle.shard_reduce([g[q0:q0 + n] for g in G]))
                               for q0, n in (z.shard_range(N, W, q) for q in range(W))]))
    torch.cuda.synchronize()
    barrier = threading.Barrier(len(ranks))
    failures = []

    def worker(r):
        try:
            torch.cuda.set_device(dev)
            s = torch.cuda.Stream()
            for t in range(1, steps + 1):
                rsds[r].copy_(torch.from_numpy(parts[t - 1]))
                torch.cuda.synchronize()
                barrier.wait()
                z.mta_step(gds[t - 1], shards[r].begin, shards[r].plan, hp_at(t), rsds[r], W, r, flags=z.STORE_G,
                           ws=wss[r], stream=s)
                try:
                    z.shard_range(10, 0, r)          # rejected: W = 0
                except z.Zero1Error as e:
                    if "W=0" not in e.message:
                        failures.append(f"rank {r}: foreign error message {e.message!r}")
                else:
                    failures.append(f"rank {r}: W = 0 accepted")
                s.synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            failures.append(f"rank {r}: {e!r}")

    threads = [threading.Thread(target=worker, args=(r,)) for r in ranks]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not failures, failures
    for r in ranks:
        o = RankState(master_full[shards[r].begin:shards[r].begin + shards[r].S])
        b, S = shards[r].begin, shards[r].S
        for t in range(1, steps + 1):
            oracle.step([g[b:b + S] for g in Gs[t - 1]], o.master, o.m, o.v, o.param, hp_at(t),
                        parts[t - 1].copy(), r)
        master, m, v, p = shards[r].gather()
        assert_f32_equal(master, o.master, f"master rank {r}")
        assert_f32_equal(m, o.m, f"m rank {r}")
        assert_f32_equal(v, o.v, f"v rank {r}")
        assert_bf16_equal(p, o.param, f"param rank {r}")


def test_empty_shard_rank(env):
    """A rank whose shard is empty (N = 10 cut into W = 8 shards of 2: ranks 5-7
    own nothing) still takes part in the step: its reduce writes a partial of
    0, its update writes the global norm and clip decision formed from every
    rank's partial and touches no element, an empty bucket's partial is 0, and
    an empty partials sum is 0."""
    torch, dev = env
    N, W = 10, 8
    G = replicas(0xE5, 1, W, N, 0.7)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    parts = np.array([oracle.sumsq(oracle.shard_reduce([g[b:b + n] for g in G]))
                      for b, n in (z.shard_range(N, W, r) for r in range(W))])
    assert [z.shard_range(N, W, r)[1] for r in range(W)] == [2, 2, 2, 2, 2, 0, 0, 0]
    ws = ws_tensor(torch, z.workspace_bytes(0, W), dev)
    rsd = torch.from_numpy(parts.copy()).to(dev)
    rsd[6] = 123.0
    b6, n6 = z.shard_range(N, W, 6)
    z.shard_reduce(gd, b6, n6, sumsq_out=rsd[6:7], ws=ws)
    info = torch.full((4,), -1.0, dtype=torch.float64, device=dev)
    sentinel = torch.full((8,), 7.0, dtype=torch.float32, device=dev)
    p16 = torch.full((8,), 0x1234, dtype=torch.int16, device=dev)
    z.adamw_step(None, gd, b6, 0, sentinel, sentinel[2:], sentinel[4:], p16, hp_at(1), rsd, W, info_out=info)
    one = torch.full((1,), 5.0, dtype=torch.float64, device=dev)
    z.partials_sum(one, 0, one)
    torch.cuda.synchronize()
    assert rsd[6].item() == 0.0
    norm = oracle.global_norm(parts)
    clip, coef = oracle.clip_coef(norm, 1.0)
    ni = info.cpu().numpy()
    assert rel_close(ni[0], float(parts.sum()), NORM_TOL) and rel_close(ni[1], norm, NORM_TOL)
    assert bool(ni[2:4].view(np.int32)[1]) == clip and ni[2:3].view(np.float32)[0] == (coef if clip else 1.0)
    assert (sentinel.cpu().numpy() == 7.0).all() and (to_np_u16(p16) == 0x1234).all()
    assert one.item() == 0.0
    # an empty bucket of a real plan: its partial is 0 and it writes nothing
    numels = [4096]
    master_full = synth.f32(4096, synth.master_key(3), 0, 0.02)
    a = MtaShard(torch, dev, numels, 1, 0, master_full)
    wsg = a.workspace(z.STORE_G)
    part = torch.full((1,), 9.0, dtype=torch.float64, device=dev)
    g1 = [to_dev_u16(torch, synth.bf16(4096, 11, 0, 0.1), dev)]
    z.mta_reduce_range([g1[0].data_ptr() + 2 * 100], a.plan, 100, 100, part, ws=wsg)
    torch.cuda.synchronize()
    assert part.item() == 0.0
