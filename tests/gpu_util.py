"""Helpers for GPU tests: device buffers for bf16 bit patterns, the mta front
end over a tensor list, and comparisons against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import zero_sharded_mixed_zero1_amd as z


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()   # raises if the HIP library is missing: never a silent fallback
    return torch


def to_dev_u16(torch, a: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def to_np_u16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def ws_tensor(torch, nbytes, dev):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def assert_f32_equal(got: np.ndarray, exp: np.ndarray, what: str):
    """Bit-exact fp32 comparison (NaN payloads aside)."""
    gb, eb = got.view(np.uint32), exp.view(np.uint32)
    nan = np.isnan(exp)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN positions differ"
    bad = np.nonzero((gb != eb) & ~nan)[0]
    if bad.size:
        k = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at {k}: "
                             f"got {got[k]!r} ({gb[k]:#010x}) expected {exp[k]!r} ({eb[k]:#010x})")


def assert_bf16_equal(got: np.ndarray, exp: np.ndarray, what: str, ulp: int = 0):
    """bf16 comparison: bit-exact (ulp=0) or within `ulp` units in the last place."""
    g = got.astype(np.int32)
    e = exp.astype(np.int32)
    gnan = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    enan = ((e & 0x7F80) == 0x7F80) & ((e & 0x7F) != 0)
    assert np.array_equal(gnan, enan), f"{what}: NaN positions differ"
    # signed-magnitude -> ordered integers
    go = np.where(g & 0x8000, -(g & 0x7FFF), g)
    eo = np.where(e & 0x8000, -(e & 0x7FFF), e)
    d = np.abs(go - eo)[~enan]
    if d.size and d.max() > ulp:
        k = int(np.nonzero(np.abs(go - eo) > ulp)[0][0])
        raise AssertionError(f"{what}: {int((d > ulp).sum())} differ by > {ulp} ulp; first at {k}: "
                             f"got {got[k]:#06x} expected {exp[k]:#06x}")


def rel_close(a: float, b: float, tol: float) -> bool:
    if np.isnan(a) or np.isnan(b):
        return np.isnan(a) and np.isnan(b)
    if np.isinf(a) or np.isinf(b):
        return a == b
    return abs(a - b) <= tol * max(abs(b), 1e-30)


class MtaShard:
    """One rank's shard on the GPU as a multi-tensor plan.

    flat_state=True: master/m/v are flat shard buffers (ZeRO-1's usual layout)
    and the pieces point into them; False: every piece gets its own buffers.
    Params are per-tensor bf16 buffers of the whole model (pieces point inside).
    """

    def __init__(self, torch, dev, numels, W, rank, master_full, mv_bf16=False, flat_state=True,
                 guard=64):
        N = sum(numels)
        self.torch, self.dev = torch, dev
        self.W, self.rank, self.numels = W, rank, list(numels)
        self.begin, self.S = z.shard_range(N, W, rank)
        self.pl = z.shard_pieces(numels, self.begin, self.begin + self.S)
        mvdt = torch.int16 if mv_bf16 else torch.float32
        self.mv_bf16 = mv_bf16
        # per-tensor bf16 params with a guard band around each, filled with a sentinel
        self.param_bufs = [torch.full((n + 2 * guard,), 0x7A5A, dtype=torch.int16, device=dev)
                           for n in numels]
        self.guard = guard
        init = master_full[self.begin:self.begin + self.S]
        if flat_state:
            self.master = torch.from_numpy(init.copy()).to(dev)
            self.m = torch.zeros(self.S, dtype=mvdt, device=dev)
            self.v = torch.zeros(self.S, dtype=mvdt, device=dev)
            self.state = [(self.master[so:so + n], self.m[so:so + n], self.v[so:so + n])
                          for _, _, so, n in self.pl]
        else:
            self.state = [(torch.from_numpy(init[so:so + n].copy()).to(dev),
                           torch.zeros(n, dtype=mvdt, device=dev), torch.zeros(n, dtype=mvdt, device=dev))
                          for _, _, so, n in self.pl]
        pieces = []
        for (ti, off, so, n), (ms, mm, vv) in zip(self.pl, self.state):
            pieces.append((n, so, self.param_bufs[ti][guard + off:], ms, mm, vv))
        self.table = ws_tensor(torch, z.mta_table_bytes(pieces), dev)
        self.plan = z.mta_plan(pieces, self.table, flags=z.MV_BF16 if mv_bf16 else 0)

    def workspace(self, flags=0):
        return ws_tensor(self.torch, z.mta_workspace_bytes(self.plan, self.W, flags), self.dev)

    def gather(self):
        """(master, m, v, param) of the shard as flat numpy arrays, plus the guard check."""
        t = self.torch
        master = t.cat([s[0] for s in self.state]).cpu().numpy()
        mvs = [t.cat([s[k] for s in self.state]).cpu().numpy() for k in (1, 2)]
        if self.mv_bf16:
            mvs = [a.view(np.uint16) for a in mvs]
        params = []
        g = self.guard
        for ti, off, so, n in self.pl:
            params.append(to_np_u16(self.param_bufs[ti][g + off:g + off + n]))
        return master, mvs[0], mvs[1], np.concatenate(params)

    def untouched_outside(self) -> bool:
        """Every param byte outside this shard's pieces still holds the sentinel."""
        g = self.guard
        covered = {}
        for ti, off, so, n in self.pl:
            covered.setdefault(ti, []).append((off, off + n))
        for ti, buf in enumerate(self.param_bufs):
            a = to_np_u16(buf)
            mask = np.ones(a.size, dtype=bool)
            for lo, hi in covered.get(ti, []):
                mask[g + lo:g + hi] = False
            if np.any(a[mask] != 0x7A5A):
                return False
        return True
