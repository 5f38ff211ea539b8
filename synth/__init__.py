"""Seeded synthetic inputs for the ZeRO-1 step: the one module both sides use.

It draws the bf16 gradients and fp32 master weights that the tests and the
bench feed to the GPU library and to the CPU oracle alike.  It holds none of the
optimizer's arithmetic.  ``synth_cpu.c`` and ``synth_gpu.hip`` implement one
counter-based definition (SplitMix64 outputs shaped into an Irwin-Hall(4)
approximation of N(0, sigma^2), optional x100 outliers, bf16 by truncation);
the definition is written out at the top of ``synth_cpu.c``.

Streams (element i is always the GLOBAL flat index, so every rank and layout
draws the same value for the same parameter):
  gradient of replica w at step t : key(seed, 1, t, w)
  fp32 master at initialisation   : key(seed, 2, 0, 0)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_CPU_SRC = os.path.join(_HERE, "synth_cpu.c")
_GPU_SRC = os.path.join(_HERE, "synth_gpu.hip")
_CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
_GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

GRAD_STREAM = 1
MASTER_STREAM = 2


def build_cpu() -> str:
    tmp = _CPU_LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-fPIC", "-shared", "-Wall", _CPU_SRC, "-o", tmp], check=True)
    os.replace(tmp, _CPU_LIB)
    return _CPU_LIB


def build_gpu() -> str:
    tmp = _GPU_LIB + ".tmp"
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-fPIC", "-shared", _GPU_SRC, "-o", tmp], check=True,
                   stderr=subprocess.PIPE)
    os.replace(tmp, _GPU_LIB)
    return _GPU_LIB


_cpu = None
_gpu = None


def cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(_CPU_LIB):
            build_cpu()
        L = ctypes.CDLL(_CPU_LIB)
        u64, i64, f32, i32, P = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_void_p)
        L.synth_at.argtypes = [u64, u64]
        L.synth_at.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64]
        L.synth_key.restype = u64
        L.synth_value.argtypes = [u64, u64, f32, i32]
        L.synth_value.restype = f32
        L.synth_fill_f32.argtypes = [P, i64, u64, u64, f32, i32]
        L.synth_fill_f32.restype = None
        L.synth_fill_bf16.argtypes = [P, i64, u64, u64, f32, i32]
        L.synth_fill_bf16.restype = None
        L.synth_gather_f32.argtypes = [P, P, i64, u64, f32, i32]
        L.synth_gather_f32.restype = None
        L.synth_gather_bf16.argtypes = [P, P, i64, u64, f32, i32]
        L.synth_gather_bf16.restype = None
        _cpu = L
    return _cpu


def gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(_GPU_LIB):
            raise RuntimeError(f"{_GPU_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_GPU_LIB)
        u64, i64, f32, i32, P = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_void_p)
        L.synth_gpu_fill_f32.argtypes = [P, i64, u64, u64, f32, i32, P]
        L.synth_gpu_fill_f32.restype = i32
        L.synth_gpu_fill_bf16.argtypes = [P, i64, u64, u64, f32, i32, P]
        L.synth_gpu_fill_bf16.restype = i32
        _gpu = L
    return _gpu


def key(seed: int, a: int, b: int = 0, c: int = 0) -> int:
    return int(cpu_lib().synth_key(seed, a, b, c))


def grad_key(seed: int, t: int, w: int) -> int:
    return key(seed, GRAD_STREAM, t, w)


def master_key(seed: int) -> int:
    return key(seed, MASTER_STREAM, 0, 0)


# ------------------------------------------------------------------ CPU draws
def f32(n: int, k: int, i0: int, sigma: float, outlier_pct: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    cpu_lib().synth_fill_f32(out.ctypes.data, n, k, i0, sigma, outlier_pct)
    return out


def bf16(n: int, k: int, i0: int, sigma: float, outlier_pct: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    cpu_lib().synth_fill_bf16(out.ctypes.data, n, k, i0, sigma, outlier_pct)
    return out


def f32_at(idx: np.ndarray, k: int, sigma: float, outlier_pct: int = 0) -> np.ndarray:
    """f32 draws at the given global indices."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    cpu_lib().synth_gather_f32(out.ctypes.data, idx.ctypes.data, idx.size, k, sigma, outlier_pct)
    return out


def bf16_at(idx: np.ndarray, k: int, sigma: float, outlier_pct: int = 0) -> np.ndarray:
    """bf16 draws at the given global indices."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    cpu_lib().synth_gather_bf16(out.ctypes.data, idx.ctypes.data, idx.size, k, sigma, outlier_pct)
    return out


# ------------------------------------------------------------------ GPU draws
def _stream_handle(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def fill_f32_(t, k: int, i0: int, sigma: float, outlier_pct: int = 0, stream=None):
    """Fill a contiguous float32 CUDA tensor in place with the same values as f32()."""
    import torch
    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
    rc = gpu_lib().synth_gpu_fill_f32(t.data_ptr(), t.numel(), k, i0, sigma, outlier_pct,
                                      _stream_handle(stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_f32 failed ({rc})")
    return t


def fill_bf16_(t, k: int, i0: int, sigma: float, outlier_pct: int = 0, stream=None):
    """Fill a contiguous 16-bit CUDA tensor (int16/uint16/bfloat16) with bf16() values."""
    import torch
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    rc = gpu_lib().synth_gpu_fill_bf16(t.data_ptr(), t.numel(), k, i0, sigma, outlier_pct,
                                       _stream_handle(stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_bf16 failed ({rc})")
    return t
