"""GPU parity at the sizes where the kernels change shape, against the CPU oracle.

The launch shape of each pass depends on the number of 2048-element tiles:
  * the sum-of-squares pass of the recompute design (W <= 4) runs on a grid
    of 6 workgroups per CU (1536) and loads U tiles together (U = 4 for W = 1,
    2; 2 for W = 3, 4) once a workgroup owns at least U tiles, i.e. once the
    shard has more tiles than U times that grid;
  * the update kernels switch from one workgroup per tile to a persistent grid
    with one contiguous part of the tiles per XCD past 8192 tiles (2^24
    elements);
  * the reduce and the fp32 sum of squares split their tiles by XCD once each
    workgroup owns 16 of them (2^26 elements at 2048 workgroups);
  * the reduce stores g non-temporally once g exceeds 128 MiB.
Every test here runs the library on shards past those thresholds, with a
ragged tail, and compares element by element with the oracle ("并行训练",
"一张卡上装了什么：混合精度与 AdamW" for the update; "训练循环与 checkpoint" for the norm
and the clip; "卡和卡怎么说话：集合通信" for the reduce): state and g bit for bit,
sums of squares to 1e-12 relative (the fp64 summation trees differ), the clip
decision and coefficient exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
import zero_sharded_mixed_zero1_amd as z
from tests.gpu_util import (assert_bf16_equal, assert_f32_equal, rel_close, to_dev_u16, to_np_u16, torch_cuda,
                            ws_tensor)

pytestmark = [pytest.mark.gpu, pytest.mark.large]

NORM_TOL = 1e-12
TILE = 2048
GRID = 2048            # the library's persistent grid: 8 workgroups per CU on 256 CUs
FEW_GRID = 1536        # its sum-of-squares pass over 1-4 slices: 6 workgroups per CU


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return torch, dev


def hp_at(t):
    return dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, step=t)


def slices(seed, t, W, S, begin, sigma):
    """The W bf16 gradient slices of one rank's shard at step t (global flat
    indices from begin), as the oracle and the GPU both see them."""
    return [synth.bf16(S, synth.grad_key(seed, t, w), begin, sigma) for w in range(W)]


# S per W: past U * 1536 tiles so every workgroup runs the U-tile loop body at
# least once (W = 1, 2: U = 4, here more than 10 tiles per workgroup, which
# also puts the update past 8192 tiles; W = 3, 4: U = 2, more than 5 tiles per
# workgroup), each with a ragged last tile
RECOMPUTE_SHARDS = {1: (1 << 25) + 777, 2: (1 << 25) + 1001, 3: (1 << 24) + 4099, 4: (1 << 24) + 2053}


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_recompute_design_multi_tile_norm_pass(env, W):
    """zero1_mta_step with the default design for W <= 4 (recompute g in the
    update), one flat tensor, 2 steps, rank 1 of W (rank 0 at W = 1): full
    state bit for bit."""
    torch, dev = env
    S = RECOMPUTE_SHARDS[W]
    rank = min(1, W - 1)
    begin = rank * S
    seed = 0x1A26E0 + W
    assert S // TILE > (4 if W <= 2 else 2) * FEW_GRID
    master0 = synth.f32(S, synth.master_key(seed), begin, 0.02)
    master = torch.from_numpy(master0.copy()).to(dev)
    m = torch.zeros(S, dtype=torch.float32, device=dev)
    v = torch.zeros(S, dtype=torch.float32, device=dev)
    params = torch.zeros(S, dtype=torch.int16, device=dev)
    table = ws_tensor(torch, z.mta_table_bytes([(S, 0, params, master, m, v)]), dev)
    plan = z.mta_plan([(S, 0, params, master, m, v)], table)
    ws = ws_tensor(torch, z.mta_workspace_bytes(plan, W), dev)
    rsd = torch.zeros(W, dtype=torch.float64, device=dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    om, ov = np.zeros(S, np.float32), np.zeros(S, np.float32)
    omaster, oparam = master0.copy(), np.zeros(S, np.uint16)
    gbuf = [torch.empty(S, dtype=torch.int16, device=dev) for _ in range(W)]
    assert z.mta_design(gbuf, 0, plan) == z.RECOMPUTE_G
    for t in (1, 2):
        G = slices(seed, t, W, S, begin, 1e-3)
        for w in range(W):
            gbuf[w].copy_(torch.from_numpy(G[w].view(np.int16)))
        rs = np.zeros(W)
        oi = oracle.step(G, omaster, om, ov, oparam, hp_at(t), rs, rank)
        z.mta_step(gbuf, 0, plan, hp_at(t), rsd, W, rank, info_out=info, ws=ws)
        torch.cuda.synchronize()
        ni = info.cpu().numpy()
        assert rel_close(rsd[rank].item(), rs[rank], NORM_TOL), (t, rsd[rank].item(), rs[rank])
        assert rel_close(ni[1], oi.norm, NORM_TOL)
        assert bool(ni[2:4].view(np.int32)[1]) == oi.clip
        assert ni[2:3].view(np.float32)[0] == oi.coef
        del G
    what = f"W={W} S={S}"
    assert_f32_equal(master.cpu().numpy(), omaster, "master " + what)
    assert_f32_equal(m.cpu().numpy(), om, "m " + what)
    assert_f32_equal(v.cpu().numpy(), ov, "v " + what)
    assert_bf16_equal(to_np_u16(params), oparam, "param " + what)


@pytest.mark.parametrize("mv_bf16", [False, True])
def test_flat_adamw_step_per_xcd_split(env, mv_bf16):
    """zero1_adamw_step with g given at 2^25 + 333 elements (16,385 tiles: the
    persistent grid with one contiguous part of the tiles per XCD), clipped,
    3 steps: full state bit for bit."""
    torch, dev = env
    S = (1 << 25) + 333
    seed = 0xF1A7
    master0 = synth.f32(S, synth.master_key(seed), 0, 0.02)
    master = torch.from_numpy(master0.copy()).to(dev)
    mvdt = torch.int16 if mv_bf16 else torch.float32
    m = torch.zeros(S, dtype=mvdt, device=dev)
    v = torch.zeros(S, dtype=mvdt, device=dev)
    params = torch.zeros(S, dtype=torch.int16, device=dev)
    info = torch.zeros(4, dtype=torch.float64, device=dev)
    npdt = np.uint16 if mv_bf16 else np.float32
    om, ov = np.zeros(S, npdt), np.zeros(S, npdt)
    omaster, oparam = master0.copy(), np.zeros(S, np.uint16)
    flags = z.MV_BF16 if mv_bf16 else 0
    for t in (1, 2, 3):
        g = synth.f32(S, synth.grad_key(seed, t, 0), 0, 1e-3 * t, 1)
        q = oracle.sumsq(g)
        rs = torch.tensor([q, 0.25], dtype=torch.float64, device=dev)     # two ranks' partials
        norm = float(np.sqrt(q + 0.25))
        clip, coef = oracle.clip_coef(norm, 1.0)
        assert clip
        sc = oracle.adamw_scalars(1e-3, 0.9, 0.95, 1e-8, 0.1, t)
        oracle.adamw(g, omaster, om, ov, oparam, sc, clip, coef)
        gd = torch.from_numpy(g).to(dev)
        z.adamw_step(gd, None, 0, S, master, m, v, params, hp_at(t), rs, 2, flags=flags, info_out=info)
        torch.cuda.synchronize()
        ni = info.cpu().numpy()
        assert ni[2:3].view(np.float32)[0] == coef and bool(ni[2:4].view(np.int32)[1])
    what = f"S={S} mv_bf16={mv_bf16}"
    assert_f32_equal(master.cpu().numpy(), omaster, "master " + what)
    if mv_bf16:
        assert_bf16_equal(to_np_u16(m), om, "m " + what)
        assert_bf16_equal(to_np_u16(v), ov, "v " + what)
    else:
        assert_f32_equal(m.cpu().numpy(), om, "m " + what)
        assert_f32_equal(v.cpu().numpy(), ov, "v " + what)
    assert_bf16_equal(to_np_u16(params), oparam, "param " + what)


def test_grad_norm_split_by_xcd(env):
    """zero1_grad_norm at 2^27 + 77 elements (65,537 tiles: 32 per workgroup,
    split by XCD), aligned and misaligned."""
    torch, dev = env
    n = (1 << 27) + 77
    x = synth.f32(n + 1, synth.key(0x6A0, 27), 0, 0.7, 1)
    ws = ws_tensor(torch, z.workspace_bytes(n, 1), dev)
    out = torch.zeros(1, dtype=torch.float64, device=dev)
    t = torch.from_numpy(x).to(dev)
    for lo in (0, 1):
        z.grad_norm(t[lo:lo + n], n, out, ws=ws)
        torch.cuda.synchronize()
        exp = oracle.sumsq(x[lo:lo + n])
        assert rel_close(out.item(), exp, NORM_TOL), (lo, out.item(), exp)


def test_shard_reduce_split_by_xcd_nontemporal_g(env):
    """zero1_shard_reduce, W = 8, at 2^26 + 5 elements (32,769 tiles: split by
    XCD; the 256 MiB fp32 g is stored non-temporally): g bit for bit, sum of
    squares to 1e-12; the norm-only call gives the same partial."""
    torch, dev = env
    W, S = 8, (1 << 26) + 5
    G = slices(0x5EDC, 1, W, S, 0, 1e-2)
    gd = [to_dev_u16(torch, g, dev) for g in G]
    ws = ws_tensor(torch, z.workspace_bytes(S, W), dev)
    g = torch.empty(S, dtype=torch.float32, device=dev)
    s1 = torch.zeros(1, dtype=torch.float64, device=dev)
    s2 = torch.zeros(1, dtype=torch.float64, device=dev)
    z.shard_reduce(gd, 0, S, g_out=g, sumsq_out=s1, ws=ws)
    z.shard_reduce(gd, 0, S, sumsq_out=s2, ws=ws)
    torch.cuda.synchronize()
    exp = oracle.shard_reduce(G)
    assert_f32_equal(g.cpu().numpy(), exp, f"g W={W} S={S}")
    q = oracle.sumsq(exp)
    assert rel_close(s1.item(), q, NORM_TOL) and s1.item() == s2.item()
