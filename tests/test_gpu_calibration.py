"""The bench's calibration kernel (libzero1_calib.so, stream_kernel) moves exactly
the bytes it claims: with one read stream and one write stream of the same
element size it is a copy of the first n_tiles * 2048 elements, for every lane
layout, tiles-in-flight count, tile order, XCD split, grid and store policy; two
read streams arrive as their XOR; nothing outside the covered range is written.
(The ceilings in the bench line are this kernel's times.)"""
from __future__ import annotations

import numpy as np
import pytest

import bench
from tests.gpu_util import torch_cuda

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return torch, dev


def run(torch, dev, rd, wr, n_tiles, grid, split, U, wide, contig):
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    bench.zcal_stream(rd, wr, n_tiles, grid, split, sink.data_ptr(), torch.cuda.current_stream().cuda_stream,
                      U, wide, contig)
    torch.cuda.synchronize()
    assert not sink.any()


@pytest.mark.parametrize("bytes_", [2, 4])
@pytest.mark.parametrize("U,contig", [(1, 0), (2, 0), (2, 1), (4, 1), (8, 0), (8, 1)])
@pytest.mark.parametrize("wide", [0, 1])
def test_calibration_pass_is_an_exact_copy(env, bytes_, U, contig, wide):
    torch, dev = env
    rng = np.random.default_rng(bytes_ * 100 + U * 10 + contig + 7 * wide)
    dt, npdt = (torch.int16, np.int16) if bytes_ == 2 else (torch.int32, np.int32)
    for n_tiles, grid, split in ((37, 16, 8), (37, 24, 1), (3001, 2048, 8), (5, 2048, 1)):
        n = n_tiles * 2048
        src_h = rng.integers(-2**15 if bytes_ == 2 else -2**31, 2**15 if bytes_ == 2 else 2**31,
                             size=n + 2 * GUARD, dtype=np.int64).astype(npdt)
        src = torch.from_numpy(src_h).to(dev)
        dst = torch.full((n + 2 * GUARD,), 0x5A5A, dtype=dt, device=dev)
        sc1 = bytes_ == 4 and grid == 24
        run(torch, dev, [(src.data_ptr() + bytes_ * GUARD, bytes_, False)],
            [(dst.data_ptr() + bytes_ * GUARD, bytes_, sc1)], n_tiles, grid, split, U, wide, contig)
        out = dst.cpu().numpy()
        what = f"bytes={bytes_} U={U} contig={contig} wide={wide} tiles={n_tiles} grid={grid} split={split}"
        assert np.array_equal(out[GUARD:GUARD + n], src_h[GUARD:GUARD + n]), what
        assert (out[:GUARD] == 0x5A5A).all() and (out[GUARD + n:] == 0x5A5A).all(), "wrote outside: " + what


def test_two_read_streams_arrive_as_their_xor(env):
    torch, dev = env
    n_tiles = 129
    n = n_tiles * 2048
    rng = np.random.default_rng(5)
    a = rng.integers(0, 2**31, size=n, dtype=np.int64).astype(np.int32)
    b = rng.integers(0, 2**31, size=n, dtype=np.int64).astype(np.int32)
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    out = torch.zeros(n, dtype=torch.int32, device=dev)
    run(torch, dev, [(ta.data_ptr(), 4, False), (tb.data_ptr(), 4, True)], [(out.data_ptr(), 4, False)],
        n_tiles, 64, 8, 2, 0, 1)
    assert np.array_equal(out.cpu().numpy(), a ^ b)


@pytest.mark.parametrize("rp,wp", [(2, 2), (0, 17), (18, 16), (16, 1)])
def test_policy_mix_moves_every_stream_exactly(env, rp, wp):
    """zcal_policy_mix (the update's stream mix with explicit cache-policy
    bits) reads every element of g, p, m, v and writes every element of p, m,
    v and out exactly once: per lane and tile, s = the xor of its four g words,
    p, m, v ^= s, out words = s; nothing outside the covered range changes."""
    torch, dev = env
    rng = np.random.default_rng(rp * 100 + wp)
    lane = np.arange(256)
    a = 512 * (lane >> 6) + 4 * (lane & 63)
    for n_tiles, grid, split in ((37, 16, 8), (3001, 2048, 8), (5, 2048, 1)):
        n = n_tiles * 2048
        host = {k: rng.integers(0, 2**32, size=(n + 2 * GUARD) // (2 if k in "go" else 1),
                                dtype=np.uint64).astype(np.uint32) for k in "gpmvo"}
        dev_t = {k: torch.from_numpy(host[k].view(np.int32).copy()).to(dev) for k in host}
        ptr = {k: dev_t[k].data_ptr() + (2 if k in "go" else 4) * GUARD for k in host}
        bench.zcal_policy_mix(rp, wp, ptr["g"], ptr["p"], ptr["m"], ptr["v"], ptr["o"], n_tiles, grid, split,
                              torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        E = (np.arange(n_tiles)[:, None] * 2048 + a[None, :]).ravel()        # element index of quad 0
        g32 = host["g"][GUARD // 2:GUARD // 2 + n // 2]
        s = g32[E // 2] ^ g32[E // 2 + 1] ^ g32[(E + 256) // 2] ^ g32[(E + 256) // 2 + 1]
        what = f"rp={rp} wp={wp} tiles={n_tiles} grid={grid} split={split}"
        for k in "pmv":
            exp = host[k].copy()
            for off in (0, 1, 2, 3, 256, 257, 258, 259):
                exp[GUARD + E + off] ^= s
            got = dev_t[k].cpu().numpy().view(np.uint32)
            assert np.array_equal(got, exp), k + " " + what
        exp = host["o"].copy()
        for w in (E // 2, E // 2 + 1, (E + 256) // 2, (E + 256) // 2 + 1):
            exp[GUARD // 2 + w] = s
        assert np.array_equal(dev_t["o"].cpu().numpy().view(np.uint32), exp), "out " + what
        assert np.array_equal(dev_t["g"].cpu().numpy().view(np.uint32), host["g"]), "g changed " + what
