"""The oracle and the library's host code built with the address and
undefined-behaviour sanitizers (CPU only, no device work).

* The oracle's C source and a small driver (tests/c/oracle_driver.c) built
  with gcc -fsanitize=address,undefined run whole steps on ragged sizes (the
  norm's 65,536-element blocks cut at odd places, W from 1 to 9, bf16 and fp32
  moments, every compatibility variant); the results must equal the regular
  oracle build bit for bit, and the sanitizers must stay silent.
* libzero1's host code built with the sanitizers on the host side only (the
  gfx950 device code is built as usual) runs tests/c/host_paths.c: the arena
  planner over many requests and every step entry point's argument checks,
  each driven to a rejection before the device is touched."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _hp(t0, max_norm):
    return dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=max_norm, step=t0)


CASES = [  # W, len, mv_bf16, variant, max_norm, steps
    (1, 1, False, 0, 1.0, 2),
    (3, 7, True, 0, 1.0, 3),
    (4, 65537, False, oracle.DECAY_FIRST, 1.0, 2),
    (9, 131071, True, oracle.CLIP_EPS, 1e9, 2),
    (8, 70000, False, oracle.G_BF16, float("inf"), 2),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_oracle_under_sanitizers(tmp_path, case):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_san"
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    os.path.join(ROOT, "oracle", "zero1_oracle.c"), os.path.join(ROOT, "tests", "c", "oracle_driver.c"),
                    "-o", str(exe), "-lm"], check=True)
    W, n, mv_bf16, variant, max_norm, steps = CASES[case]
    seed = 0x5A40 + case
    t0 = 1 + 7 * case
    n_ranks, my_rank = 3, 1
    rs0 = np.array([0.25, 0.0, 4.0], dtype=np.float64)
    master0 = synth.f32(n, synth.master_key(seed), 0, 0.02)
    grads = [[synth.bf16(n, synth.grad_key(seed, t0 + k, w), 0, 0.05, 1) for w in range(W)] for k in range(steps)]
    hp = _hp(t0, max_norm)
    with open(tmp_path / "case.bin", "wb") as f:
        np.array([W, int(mv_bf16), variant, steps, n_ranks, my_rank], dtype=np.int32).tofile(f)
        np.array([n, t0], dtype=np.int64).tofile(f)
        np.array([hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["max_norm"]],
                 dtype=np.float64).tofile(f)
        rs0.tofile(f)
        master0.tofile(f)
        for gs in grads:
            for g in gs:
                g.astype(np.uint16).tofile(f)
    out = subprocess.run([str(exe), str(tmp_path / "case.bin"), str(tmp_path / "out.bin")],
                         capture_output=True, text=True, timeout=300, env=SAN_ENV)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "runtime error" not in out.stderr and "AddressSanitizer" not in out.stderr, out.stderr

    mvdt = np.uint16 if mv_bf16 else np.float32
    master, m, v = master0.copy(), np.zeros(n, mvdt), np.zeros(n, mvdt)
    param, rs = np.zeros(n, np.uint16), rs0.copy()
    infos = []
    for k in range(steps):
        i = oracle.step(grads[k], master, m, v, param, _hp(t0 + k, max_norm), rs, my_rank, variant=variant)
        infos.append([i.norm, i.coef, float(i.clip), rs[my_rank]])
    raw = open(tmp_path / "out.bin", "rb").read()
    o = 0
    got_info = np.frombuffer(raw, np.float64, 4 * steps, o); o += 32 * steps
    got_master = np.frombuffer(raw, np.float32, n, o); o += 4 * n
    mvb = 2 if mv_bf16 else 4
    got_m = np.frombuffer(raw, mvdt, n, o); o += mvb * n
    got_v = np.frombuffer(raw, mvdt, n, o); o += mvb * n
    got_p = np.frombuffer(raw, np.uint16, n, o); o += 2 * n
    assert o == len(raw)
    np.testing.assert_array_equal(got_info.view(np.uint64), np.array(infos, np.float64).reshape(-1).view(np.uint64))
    for a, b, name in ((got_master, master, "master"), (got_m, m, "m"), (got_v, v, "v"), (got_p, param, "param")):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name


def test_host_library_under_sanitizers(tmp_path):
    hipcc, clang = "/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("no hipcc/clang")
    csrc = os.path.join(ROOT, "zero_sharded_mixed_zero1_amd", "csrc")
    lib = tmp_path / "libzero1_san.so"
    # the sanitizers instrument the host side only; the device code is built as usual
    subprocess.run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
                    "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), os.path.join(csrc, "api.cpp"), os.path.join(csrc, "kernels.hip"),
                    "-o", str(lib)], check=True, capture_output=True)
    # the host code really is instrumented: the library calls the sanitizers' runtime
    syms = subprocess.run(["nm", "-D", "--undefined-only", str(lib)], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    exe = tmp_path / "host_paths"
    subprocess.run([clang, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "host_paths.c"),
                    "-o", str(exe), "-L", str(tmp_path), "-lzero1_san", f"-Wl,-rpath,{tmp_path}", "-lm"], check=True)
    # the HIP runtime library the host code links keeps allocations of its own until exit
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0, out.stdout[-4000:] + out.stderr[-4000:]
    assert out.stdout.strip().endswith("all ok"), out.stdout[-4000:]
    assert "runtime error" not in out.stderr and "AddressSanitizer" not in out.stderr, out.stderr[-4000:]


@pytest.mark.parametrize("compiler", ["gcc", "/opt/rocm/llvm/bin/clang"])
def test_sanitizer_toolchain_reports_a_planted_overflow(tmp_path, compiler):
    """The flags used above do catch an error: a one-element heap overflow in
    a throwaway C program built the same way aborts with a report."""
    cc = shutil.which(compiler) or (compiler if os.path.exists(compiler) else None)
    if cc is None:
        pytest.skip(f"no {compiler}")
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint main(int c, char** v) { (void)v; int* a = malloc(4 * sizeof(int));"
                   " a[3 + c] = 1; int r = a[0]; free(a); return r; }\n")
    exe = tmp_path / "planted"
    subprocess.run([cc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60, env=SAN_ENV)
    reported = "heap-buffer-overflow" in out.stderr or "insufficient space" in out.stderr
    assert out.returncode != 0 and reported, out.stderr[-2000:]
