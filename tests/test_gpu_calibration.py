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
