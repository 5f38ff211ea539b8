"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/zero1.h declares, and rejects bad arguments before it
touches the device.  Also the host layout helpers."""
from __future__ import annotations

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
    # header, library and binding agree on the ABI version
    src = open(os.path.join(ROOT, "include", "zero1.h")).read()
    header = int(re.search(r"#define ZERO1_ABI_VERSION (\d+)", src).group(1))
    from zero_sharded_mixed_zero1_amd import binding
    assert z.abi_version() == header == binding.ABI_VERSION


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
    # 0x10 belonged to a single-launch design that is no longer in the library
    plan = z.Plan(table=FAKE, shard_len=1000, n_pieces=1, n_chunks=1, chunk_elems=2048)
    assert "unknown flag" in _einval(lambda: z.mta_step(g, 0, plan, _hp(), FAKE, 2, 0, flags=0x10,
                                                        ws=FAKE, ws_bytes=1 << 30, stream=0))


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


# ---------------------------------------------------------------- arena planner
GiB = 1 << 30
UNIT = 2 << 20


def _arena_intervals(L, req_W, S, grad_elems, param_elems, mvb, store_g):
    iv = [("ws", L.ws, L.ws + L.ws_bytes), ("master", L.master, L.master + 4 * S),
          ("m", L.m, L.m + mvb * S), ("v", L.v, L.v + mvb * S),
          ("params", L.params, L.params + 2 * param_elems)]
    iv += [(f"grads[{w}]", L.grads[w], L.grads[w] + 2 * grad_elems) for w in range(req_W)]
    return iv


@pytest.mark.parametrize("S,W,ge,go,pe,po,flags", [
    (15554976, 8, 124439808, 4 * 15554976, 124439808, 4 * 15554976, 0),          # GPT-2 small, full replicas
    (842301952, 8, 842301952, 0, 6738415616, 3 * 842301952, 0),                   # Llama-7B/8 rank 3
    (117187500, 64, 117187500, 0, 7_500_000_000, 0, 0),                            # 7.5e9/64 rank 0
    (7_000_000_000, 1, 7_000_000_000, 0, 7_000_000_000, 0, z.MV_BF16),             # 7e9 W=1 bf16 m,v
    (262144, 4, 1 << 20, 0, 1 << 20, 0, z.RECOMPUTE_G),                            # 2^20 W=4, rank 0
    (1000, 3, 5000, 1234, 7000, 99, z.STORE_G),
    (1000, 3, 5000, 1234, 7000, 99, z.RECOMPUTE_G | z.MV_BF16),
])
def test_arena_plan_layout(S, W, ge, go, pe, po, flags):
    for cap in (1 << 62, None):
        if cap is None:   # a capacity that forces a smaller spacing
            full = z.arena_plan(S, W, ge, go, pe, po, flags)
            cap = full.total_bytes - 4 * (full.spacing // 3)
            if full.spacing > 40 * GiB:
                # the arrays themselves set the spacing: nothing smaller fits
                assert "packed layout" in _einval(lambda: z.arena_plan(S, W, ge, go, pe, po, flags, capacity=cap))
                continue
        L = z.arena_plan(S, W, ge, go, pe, po, flags, capacity=cap)
        store_g = bool(flags & z.STORE_G) or (not (flags & z.RECOMPUTE_G) and W > 4)
        mvb = 2 if flags & z.MV_BF16 else 4
        assert L.total_bytes <= cap
        assert L.ws_bytes == z.lib().zero1_workspace_bytes(S, W, z.STORE_G if store_g else 0)
        iv = _arena_intervals(L, W, S, ge, pe, mvb, store_g)
        for name, a, b in iv:
            assert 0 <= a < b <= L.total_bytes, name
        iv.sort(key=lambda x: x[1])
        for (n1, a1, b1), (n2, a2, b2) in zip(iv, iv[1:]):
            assert b1 <= a2, f"{n1} overlaps {n2}"
        # the five spaced shard starts sit at base + k D, on 2 MiB boundaries
        base = L.ws if store_g else L.grads[0] + 2 * go
        starts = [base, L.master, L.m, L.v, L.params + 2 * po]
        assert all(x % UNIT == 0 for x in starts) and L.spacing % UNIT == 0
        assert starts == [base + k * L.spacing for k in range(5)]
        if cap == 1 << 62:
            assert L.spacing >= 40 * GiB
        else:
            assert L.spacing < full.spacing
        # the remaining buffers start on 2 MiB boundaries
        for w in range(0 if store_g else 1, W):
            assert L.grads[w] % UNIT == 0
        if not store_g:
            assert L.ws % UNIT == 0


def test_arena_plan_rejects():
    msg = _einval(lambda: z.arena_plan(0, 8, 10, 0, 10, 0))
    assert "shard_len" in msg
    assert "W=0" in _einval(lambda: z.arena_plan(10, 0, 10, 0, 10, 0))
    assert "W=129" in _einval(lambda: z.arena_plan(10, 129, 10, 0, 10, 0))
    assert "gradient buffers" in _einval(lambda: z.arena_plan(10, 2, 15, 6, 10, 0))
    assert "parameter buffer" in _einval(lambda: z.arena_plan(10, 2, 10, 0, 19, 10))
    assert "exclusive" in _einval(lambda: z.arena_plan(10, 2, 10, 0, 10, 0, z.STORE_G | z.RECOMPUTE_G))
    # flags that do not concern the layout are ignored
    assert z.arena_plan(10, 2, 10, 0, 10, 0, z.DECAY_FIRST).total_bytes == z.arena_plan(10, 2, 10, 0, 10, 0).total_bytes
    assert "unknown" in _einval(lambda: z.arena_plan(10, 2, 10, 0, 10, 0, 1 << 24))
    assert "capacity" in _einval(lambda: z.arena_plan(1 << 20, 8, 1 << 20, 0, 1 << 20, 0, 0, capacity=1 << 20))


# ---------------------------------------------------------------- device step scalars
def test_step_scalars_derive_matches_the_oracle():
    """The host derivation of the per-step fp32 scalars (what every step call
    passes to its kernels, and what a graph replay reads from device memory)
    equals the oracle's, over a sweep of t, lr and betas."""
    import oracle
    for t in (1, 2, 3, 10, 1000, 10 ** 6):
        for lr, b1, b2, eps, wd in [(1e-3, 0.9, 0.95, 1e-8, 0.1), (3e-4, 0.8, 0.999, 1e-6, 0.0),
                                    (0.1, 0.0, 0.5, 0.0, 1.0), (6e-4, 0.9, 0.95, 1e-8, 0.01)]:
            s = z.step_scalars_derive(dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd,
                                           max_norm=0.5, step=t))
            o = oracle.adamw_scalars(lr, b1, b2, eps, wd, t)
            got = [s.beta1, s.beta2, s.one_minus_beta1, s.one_minus_beta2, s.eps, s.step_size, s.decay]
            exp = [o.b1, o.b2, o.a1, o.a2, o.eps, o.sigma, o.delta]
            assert got == exp, (t, lr, got, exp)
            assert s.max_norm == 0.5 and s.reserved == 0.0
    assert "step=0" in _einval(lambda: z.step_scalars_derive(_hp(step=0)))
    assert "beta1" in _einval(lambda: z.step_scalars_derive(_hp(beta1=1.0)))


def test_device_scalars_must_be_aligned():
    bufs = [FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20)]
    hp = z.HParams(0, 0, 0, 0, 0, 0, 0, FAKE + 4)
    assert "aligned" in _einval(lambda: z.adamw_step(FAKE + (4 << 20), None, 0, 100, *bufs, hp,
                                                     FAKE + (5 << 20), 1, stream=0))


def test_c_consumer_compiles_and_links(tmp_path):
    """include/zero1.h is valid C11 and libzero1.so links from C: a small C
    program calls the host-only entry points (no device work)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    libdir = os.path.dirname(z.lib_path)
    exe = tmp_path / "abi_consumer"
    src = os.path.join(ROOT, "tests", "c", "abi_consumer.c")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-o", str(exe), "-L", libdir, "-lzero1", f"-Wl,-rpath,{libdir}", "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("all ok"), out.stdout


def test_bench_entry_points_and_gpu_count_contract():
    """bench.py keeps its step machinery, and --gpus N > 1 exits with a message
    (one GPU is measured) before touching any device."""
    import subprocess
    import sys
    import bench
    for name in ("setup", "run_steps", "measure", "calibrated", "calibrate", "cpu_baseline", "bucketed_timing",
                 "summarize_pmc", "summarize_kt", "traffic_from_summary", "kernel_source_hash", "other_tensors",
                 "main"):
        assert callable(getattr(bench, name)), name
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 2 and "ONE GPU" in out.stderr, (out.returncode, out.stderr)
    assert out.stdout == ""


def test_profile_summaries_from_counter_and_trace_files(tmp_path):
    """The profile summarizers: counter bytes per dispatch scaled by the plain
    copy's reading, the bench's traffic read back only while the kernel source
    hash matches, and kernel-trace statistics split by grid size."""
    import bench
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    for d, counts in ((fetch, {"upd": [100.0, 102.0, 101.0], "red": [40.0, 40.0, 40.0], "neg": [524288.0]}),
                      (write, {"upd": [70.0, 70.0, 70.0], "red": [10.0, 12.0, 11.0], "neg": [1048576.0]})):
        (d / "x").mkdir(parents=True)
        names = {"upd": "void z1::adamw_mta_kernel<true, 0, false>(float const*)",
                 "red": "void z1::reduce_kernel<true, true, true, false, 0>(z1::Reduce)",
                 "neg": "void at::native::neg_kernel_impl(float)"}
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        disp = 0
        for key, vals in counts.items():
            for v in vals:
                disp += 1
                # two rows (e.g. two counter instances) of one dispatch add up
                rows.append(f'{disp},"{names[key]}",C,{v / 2}')
                rows.append(f'{disp},"{names[key]}",C,{v / 2}')
        (d / "x" / "pmc_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "summary.txt"
    bench.summarize_pmc(str(fetch), str(write), str(out))
    kv = dict(l.split(" = ", 1) for l in out.read_text().splitlines() if " = " in l and not l.startswith("#"))
    # fetch scale: 1 GiB / (524288 KiB) = x2; write scale x1; medians 101 / 70 and 40 / 11 KiB
    assert int(kv["update_fetch_bytes"]) == 101 * 1024 * 2 and int(kv["update_write_bytes"]) == 70 * 1024
    assert int(kv["reduce_fetch_bytes"]) == 40 * 1024 * 2 and int(kv["reduce_write_bytes"]) == 11 * 1024
    assert bench.traffic_from_summary(str(out), "update") == 101 * 2048 + 70 * 1024
    assert bench.traffic_from_summary(str(out), "reduce") == 40 * 2048 + 11 * 1024
    stale = tmp_path / "stale.txt"
    stale.write_text(out.read_text().replace(bench.kernel_source_hash(), "0" * 16))
    assert bench.traffic_from_summary(str(stale), "update") is None
    # kernel trace: two grids of one kernel are reported apart
    kt = tmp_path / "kt" / "x"
    kt.mkdir(parents=True)
    rows = ["Kernel_Name,Grid_Size_X,Workgroup_Size_X,Start_Timestamp,End_Timestamp"]
    for i, (grid, dur) in enumerate([(2048, 50000), (2048, 52000), (768, 9000)]):
        rows.append(f'"void z1::(anonymous namespace)::reduce_kernel<true>(z1::Reduce)",{grid * 256},256,'
                    f'{1000 * i},{1000 * i + dur}')
    (kt / "kt_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    kout = tmp_path / "kt.txt"
    bench.summarize_kt(str(tmp_path / "kt"), str(kout))
    lines = [l for l in kout.read_text().splitlines() if l.startswith("reduce_kernel")]
    assert len(lines) == 2
    cols = [[c.strip() for c in l.split("|")] for l in lines]
    assert cols[0][1:4] == ["2048", "2", "51.00"] and cols[1][1:4] == ["768", "1", "9.00"]


def test_bench_arena_gaps():
    """The bench's gap finder returns exactly the byte ranges of the arena that
    no array occupies (overlapping and touching spans merged, small gaps and
    the space before, between and after the arrays handled alike)."""
    import bench

    class Arena:
        def __init__(self, n):
            self.n = n

        def numel(self):
            return self.n

    st = {"arena": Arena(1000), "spans": [(0, 100), (50, 120), (120, 300), (305, 400), (700, 900)]}
    assert bench.arena_gaps(st, min_bytes=1) == [(300, 305), (400, 700), (900, 1000)]
    assert bench.arena_gaps(st, min_bytes=10) == [(400, 700), (900, 1000)]
    st = {"arena": Arena(500), "spans": [(100, 200)]}
    assert bench.arena_gaps(st, min_bytes=1) == [(0, 100), (200, 500)]
    st = {"arena": Arena(200), "spans": [(0, 200)]}
    assert bench.arena_gaps(st, min_bytes=1) == []


def test_arena_tensors_views():
    """arena_tensors (CPU memory here: the planner is host code) gives views of
    the right type and length at the planner's offsets from a 2 MiB-aligned
    base: the spaced arrays' shard starts on 2 MiB boundaries, no two arrays
    overlapping, everything inside the one allocation."""
    import torch
    import zero_sharded_mixed_zero1_amd as z
    S, W, N, b = 5000, 3, 15000, 5000
    for flags in (z.STORE_G, z.RECOMPUTE_G | z.MV_BF16, 0):
        a = z.arena_tensors(S, W, N, b, N, b, flags=flags, device="cpu", capacity=256 << 20)
        L = a.layout
        assert L.total_bytes <= 256 << 20 and a.storage.numel() == L.total_bytes + (2 << 20)
        base = a.storage.data_ptr() + a.base
        assert base % (2 << 20) == 0
        mv = torch.int16 if flags & z.MV_BF16 else torch.float32
        assert a.master.dtype == torch.float32 and a.master.numel() == S
        assert a.m.dtype == mv and a.v.dtype == mv and a.m.numel() == S and a.v.numel() == S
        assert a.params.dtype == torch.int16 and a.params.numel() == N
        assert len(a.grads) == W and all(g.dtype == torch.int16 and g.numel() == N for g in a.grads)
        assert a.ws.numel() == L.ws_bytes == z.mta_workspace_bytes(
            z.Plan(shard_len=S), W, flags & (z.STORE_G | z.RECOMPUTE_G))
        for t, off in ((a.master, L.master), (a.m, L.m), (a.v, L.v), (a.params, L.params), (a.ws, L.ws)):
            assert t.data_ptr() == base + off
        starts = [a.master.data_ptr(), a.m.data_ptr(), a.v.data_ptr(), a.params.data_ptr() + 2 * b]
        starts.append(a.ws.data_ptr() if flags & z.STORE_G or (not flags & z.RECOMPUTE_G and W > 4)
                      else a.grads[0].data_ptr() + 2 * b)
        assert all(p % (2 << 20) == 0 for p in starts), [p % (2 << 20) for p in starts]
        spans = sorted((t.data_ptr(), t.data_ptr() + t.numel() * t.element_size())
                       for t in [a.ws, a.master, a.m, a.v, a.params] + a.grads)
        assert all(e0 <= s1 for (_, e0), (s1, _) in zip(spans, spans[1:])), spans
        lo, hi = a.storage.data_ptr(), a.storage.data_ptr() + a.storage.numel()
        assert lo <= spans[0][0] and spans[-1][1] <= hi
