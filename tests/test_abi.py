"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/zero1.h declares, and rejects bad arguments before it
touches the device.  Also the host layout helpers."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

import zero_sharded_mixed_zero1_amd as z
from synth.workloads import configs, gpt2_small_tensors, llama_7b_tensors, shard_range

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "zero1.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zero1_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    L = z.lib()
    for n in names:
        assert hasattr(L, n), f"libzero1.so does not export {n}"
    assert z.abi_version() == 1


def test_oracle_and_synth_libraries_load():
    import oracle
    import synth
    assert oracle.lib() is not None and synth.cpu_lib() is not None


def test_status_strings():
    L = z.lib()
    assert L.zero1_status_string(0) == b"ZERO1_OK"
    assert L.zero1_status_string(1) == b"ZERO1_EINVAL"
    assert L.zero1_status_string(99) == b"ZERO1_UNKNOWN"


@pytest.mark.parametrize("n,W", [(10, 4), (7, 8), (1 << 20, 4), (124_439_808, 8), (0, 3), (5, 1)])
def test_shard_range_matches_convention(n, W):
    covered = 0
    for r in range(W):
        b, l = z.shard_range(n, W, r)
        assert (b, b + l) == shard_range(n, W, r)
        assert b == min(covered, n)
        covered = b + l
    assert covered == n


def test_shard_range_errors():
    for args in [(-1, 2, 0), (10, 0, 0), (10, 2, 2), (10, 2, -1)]:
        with pytest.raises(z.Zero1Error) as e:
            z.shard_range(*args)
        assert e.value.name == "ZERO1_EINVAL"


def test_workspace_bytes():
    base = z.workspace_bytes(0, 4, 0)
    assert base % 256 == 0 and base >= 256 + 8 * 1024
    assert z.workspace_bytes(1000, 8, z.STORE_G) == base + 4096
    assert z.workspace_bytes(1000, 8, 0) == base


FAKE = 1 << 40      # a device-looking address; validation must fail before any use


def _hp(**kw):
    d = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, step=1)
    d.update(kw)
    return d


def _einval(fn):
    with pytest.raises(z.Zero1Error) as e:
        fn()
    assert e.value.name == "ZERO1_EINVAL", e.value
    return e.value.message


def test_shard_reduce_rejects_bad_arguments():
    g = [FAKE + 4096 * k for k in range(4)]
    assert "W=0" in _einval(lambda: z.shard_reduce([], 0, 10, g_out=FAKE, stream=0))
    assert "W=129" in _einval(lambda: z.shard_reduce([FAKE] * 129, 0, 10, g_out=FAKE, stream=0))
    assert "negative" in _einval(lambda: z.shard_reduce(g, 0, -1, g_out=FAKE, stream=0))
    assert "negative" in _einval(lambda: z.shard_reduce(g, -3, 10, g_out=FAKE, stream=0))
    assert "grads[2]" in _einval(lambda: z.shard_reduce([FAKE, FAKE, 0, FAKE], 0, 10, g_out=FAKE, stream=0))
    assert "both NULL" in _einval(lambda: z.shard_reduce(g, 0, 10, stream=0))
    # g_out overlapping a gradient slice
    assert "overlap" in _einval(lambda: z.shard_reduce(g, 0, 1000, g_out=g[1] + 8, stream=0))


def test_adamw_step_rejects_bad_hparams():
    bufs = [FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20)]
    def call(**kw):
        return lambda: z.adamw_step(FAKE + (4 << 20), None, 0, 100, *bufs, _hp(**kw), FAKE + (5 << 20),
                                    1, stream=0)
    assert "step=0" in _einval(call(step=0))
    assert "beta1" in _einval(call(beta1=1.0))
    assert "beta2" in _einval(call(beta2=-0.1))
    assert "lr" in _einval(call(lr=-1.0))
    assert "lr" in _einval(call(lr=math.nan))
    assert "eps" in _einval(call(eps=-1e-8))
    assert "weight_decay" in _einval(call(weight_decay=-0.1))
    assert "max_norm" in _einval(call(max_norm=0.0))
    assert "max_norm" in _einval(call(max_norm=math.nan))
    assert "n_ranks" in _einval(lambda: z.adamw_step(FAKE + (4 << 20), None, 0, 100, *bufs, _hp(),
                                                     FAKE + (5 << 20), 0, stream=0))
    # overlapping state buffers
    assert "overlap" in _einval(lambda: z.adamw_step(FAKE + (4 << 20), None, 0, 100, FAKE, FAKE + 200,
                                                     bufs[2], bufs[3], _hp(), FAKE + (5 << 20), 1, stream=0))


def test_mta_plan_rejects_bad_piece_lists():
    def pc(n, off, base):
        return (n, off, base, base + (1 << 20), base + (2 << 20), base + (3 << 20))
    # gap between pieces
    assert "tile" in _einval(lambda: z.mta_plan([pc(10, 0, FAKE), pc(10, 11, FAKE + (8 << 20))], FAKE, 1 << 16))
    # overlap in shard positions
    assert "tile" in _einval(lambda: z.mta_plan([pc(10, 0, FAKE), pc(10, 5, FAKE + (8 << 20))], FAKE, 1 << 16))
    # does not start at 0
    assert "tile" in _einval(lambda: z.mta_plan([pc(10, 3, FAKE)], FAKE, 1 << 16))
    # zero-sized piece
    assert "numel" in _einval(lambda: z.mta_plan([pc(0, 0, FAKE)], FAKE, 1 << 16))
    # two pieces sharing a master buffer
    assert "overlap" in _einval(lambda: z.mta_plan([pc(10, 0, FAKE), pc(10, 10, FAKE + 16)], FAKE, 1 << 16))
    assert "at least one" in _einval(lambda: z.mta_plan([], FAKE, 1 << 16))


def test_mta_table_bytes():
    p = [(2048 * 3 + 1, 0, FAKE, FAKE, FAKE, FAKE), (5, 2048 * 3 + 1, FAKE, FAKE, FAKE, FAKE)]
    assert z.mta_table_bytes(p) == 256 + 16 * (4 + 1)


def test_shard_pieces_tile_each_shard():
    for name, tensors, W in [("gpt2", gpt2_small_tensors(), 8), ("llama", llama_7b_tensors(), 8)]:
        numels = [n for _, n in tensors]
        N = sum(numels)
        for r in range(W):
            b, e = shard_range(N, W, r)
            ps = z.shard_pieces(numels, b, e)
            pos = 0
            for ti, off, so, n in ps:
                assert so == pos and n > 0 and off + n <= numels[ti]
                assert sum(numels[:ti]) + off == b + so
                pos += n
            assert pos == e - b


def test_workload_shapes():
    c = configs()
    assert c["C2"].n_total == 124_439_808 and len(c["C2"].tensors) == 148
    assert c["C2"].S == 15_554_976
    assert c["C4"].n_total == 6_738_415_616 and len(c["C4"].tensors) == 291
    assert c["C4"].S == 842_301_952
    assert c["C3"].S == 117_187_500
    numels = [n for _, n in c["C2"].tensors]
    b, e = c["C2"].shard
    ps = z.shard_pieces(numels, b, e)
    assert len(ps) == 31 and min(p[3] for p in ps) == 768
    numels = [n for _, n in c["C4"].tensors]
    b, e = c["C4"].shard
    ps = z.shard_pieces(numels, b, e)
    assert len(ps) == 40 and min(p[3] for p in ps) == 2048
    assert all(p[2] % 8 == 0 and p[3] % 8 == 0 for p in ps)


def test_unknown_flags_are_rejected():
    g = [FAKE + 4096 * k for k in range(2)]
    assert "unknown flag" in _einval(lambda: z.shard_reduce(g, 0, 10, g_out=FAKE + (1 << 30), flags=0x1000, stream=0))
    bufs = [FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20)]
    assert "unknown flag" in _einval(lambda: z.adamw_step(FAKE + (4 << 20), None, 0, 100, *bufs, _hp(),
                                                          FAKE + (5 << 20), 1, flags=0x100, stream=0))


def test_bucketed_reduction_rejects_bad_arguments():
    plan = z.Plan(table=FAKE, shard_len=1000, n_pieces=1, n_chunks=1, chunk_elems=2048)
    g = [FAKE + (1 << 20) * k for k in range(4)]
    assert "inside the shard" in _einval(lambda: z.mta_reduce_range(g, plan, 5, 3, FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "inside the shard" in _einval(lambda: z.mta_reduce_range(g, plan, -1, 3, FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "inside the shard" in _einval(lambda: z.mta_reduce_range(g, plan, 0, 1001, FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "STORE_G only" in _einval(lambda: z.mta_reduce_range(g, plan, 0, 10, FAKE, flags=z.RECOMPUTE_G,
                                                                ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "sumsq_out" in _einval(lambda: z.mta_reduce_range(g, plan, 0, 10, 0, ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "plan" in _einval(lambda: z.mta_reduce_range(g, z.Plan(), 0, 10, FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "W=0" in _einval(lambda: z.mta_reduce_range([], plan, 0, 10, FAKE, ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "unknown" in _einval(lambda: z.mta_reduce_range(g, plan, 0, 10, FAKE, flags=1 << 20,
                                                           ws=FAKE, ws_bytes=1 << 30, stream=0))
    assert "n=" in _einval(lambda: z.partials_sum(FAKE, -1, FAKE, stream=0))
    assert "n=" in _einval(lambda: z.partials_sum(FAKE, 8193, FAKE, stream=0))
    assert "NULL" in _einval(lambda: z.partials_sum(FAKE, 4, 0, stream=0))
