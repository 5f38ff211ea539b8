"""zero1_mta_step_static (the step with its workspace in the library's static
device array, for callers that cannot allocate) against zero1_mta_step with a
caller's workspace: two calls in a row on one GPU, the second on a smaller
shard (other pieces, other length), both designs; master, m, v, bf16 params,
this rank's partial and the norm info must be identical bit for bit.  Plus the
host-side refusal of a store-g shard longer than the array holds."""
from __future__ import annotations

import numpy as np
import pytest

import synth
import zero_sharded_mixed_zero1_amd as z
from tests.gpu_util import MtaShard, assert_bf16_equal, assert_f32_equal, to_dev_u16

FAKE = 1 << 44


def hp_at(t):
    return dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, step=t)


def test_static_step_refuses_a_shard_beyond_the_array():
    plan = z.Plan(table=FAKE, shard_len=z.STATIC_MAX_G_ELEMS + 1, n_pieces=1, n_chunks=1, chunk_elems=2048)
    g = [FAKE + (1 << 36) * k for k in range(8)]
    with pytest.raises(z.Zero1Error) as e:
        z.mta_step_static(g, 0, plan, hp_at(1), FAKE, 8, 0, stream=0)
    assert e.value.name == "ZERO1_EINVAL" and "static scratch" in e.value.message


@pytest.mark.gpu
@pytest.mark.parametrize("W,design", [(8, z.STORE_G), (3, z.RECOMPUTE_G), (8, 0)])
def test_static_step_matches_workspace_step(W, design):
    from tests.gpu_util import torch_cuda
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # call 1: a ragged list whose rank-2 shard is about 1.3M elements; call 2:
    # another list whose shard is about 60k elements (what call 1 left in the
    # array must not leak into call 2)
    for call, (numels, rank, t) in enumerate([([400_001, 3, 2_048 * 900 + 17, 1_000_000 + 5, 768] * 2, 2, 1),
                                              ([70_001, 9, 64_000 + 3, 50_000], 1, 2)]):
        N = sum(numels)
        seed = 0x57A7 + call
        master_full = synth.f32(N, synth.master_key(seed), 0, 0.02)
        a = MtaShard(torch, dev, numels, W, rank, master_full)
        b = MtaShard(torch, dev, numels, W, rank, master_full)
        G = [synth.bf16(N, synth.grad_key(seed, t, w), 0, 0.02, 1) for w in range(W)]
        gd = [to_dev_u16(torch, x, dev) for x in G]
        rs_a = torch.full((W,), 0.3, dtype=torch.float64, device=dev)
        rs_b = rs_a.clone()
        ia = torch.zeros(4, dtype=torch.float64, device=dev)
        ib = torch.zeros(4, dtype=torch.float64, device=dev)
        ws = a.workspace(design)
        for step in range(t, t + 2):
            z.mta_step(gd, a.begin, a.plan, hp_at(step), rs_a, W, rank, flags=design, info_out=ia, ws=ws)
            z.mta_step_static(gd, b.begin, b.plan, hp_at(step), rs_b, W, rank, flags=design, info_out=ib)
        torch.cuda.synchronize()
        what = f"call {call + 1} W={W} design={design} S={a.S}"
        assert rs_a.cpu().numpy().tobytes() == rs_b.cpu().numpy().tobytes(), what
        assert ia.cpu().numpy().tobytes() == ib.cpu().numpy().tobytes(), what
        ga, gb = a.gather(), b.gather()
        for k, name in ((0, "master"), (1, "m"), (2, "v")):
            assert_f32_equal(gb[k], ga[k], f"{name} static vs workspace, {what}")
        assert_bf16_equal(gb[3], ga[3], f"param static vs workspace, {what}")
        assert b.untouched_outside(), what
        assert np.isfinite(gb[0]).all()


@pytest.mark.gpu
def test_static_step_replays_from_a_captured_graph():
    """The use the entry point is for: after one eager call on the device,
    the step is captured into a HIP graph without a workspace and replayed
    three times, with eager work between the replays; each replay equals a
    zero1_mta_step call with a caller's workspace, bit for bit."""
    from tests.gpu_util import torch_cuda
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W, rank = 8, 5
    numels = [300_001, 7, 2_048 * 50 + 9, 90_000]
    N = sum(numels)
    master_full = synth.f32(N, synth.master_key(0x6A9), 0, 0.02)
    a = MtaShard(torch, dev, numels, W, rank, master_full)
    b = MtaShard(torch, dev, numels, W, rank, master_full)
    G = [synth.bf16(N, synth.grad_key(0x6A9, 1, w), 0, 0.02, 1) for w in range(W)]
    gd = [to_dev_u16(torch, x, dev) for x in G]
    rs_a = torch.full((W,), 0.3, dtype=torch.float64, device=dev)
    rs_b = rs_a.clone()
    ia = torch.zeros(4, dtype=torch.float64, device=dev)
    ib = torch.zeros(4, dtype=torch.float64, device=dev)
    ws = a.workspace()
    # the eager first call on this device (looks the array up)
    z.mta_step(gd, a.begin, a.plan, hp_at(1), rs_a, W, rank, info_out=ia, ws=ws)
    z.mta_step_static(gd, b.begin, b.plan, hp_at(1), rs_b, W, rank, info_out=ib)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        z.mta_step_static(gd, b.begin, b.plan, hp_at(2), rs_b, W, rank, info_out=ib)
    torch.cuda.synchronize()
    scratch = torch.ones(1 << 20, device=dev)
    for k in range(3):
        z.mta_step(gd, a.begin, a.plan, hp_at(2), rs_a, W, rank, info_out=ia, ws=ws)
        graph.replay()
        scratch.mul_(1.0001).add_(1.0)
        torch.cuda.synchronize()
        ga, gb = a.gather(), b.gather()
        for j, name in ((0, "master"), (1, "m"), (2, "v")):
            assert_f32_equal(gb[j], ga[j], f"{name} replay {k}")
        assert_bf16_equal(gb[3], ga[3], f"param replay {k}")
        assert ia.cpu().numpy().tobytes() == ib.cpu().numpy().tobytes()
        assert rs_a.cpu().numpy().tobytes() == rs_b.cpu().numpy().tobytes()
    del graph
