"""Plain CPU oracle for one rank's ZeRO-1 optimizer step (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this module to obtain the values the
GPU library must reproduce.  The product package never imports it, and it
shares no code with the GPU library.

The arithmetic lives in ``zero1_oracle.c`` (plain C, built with
``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals numpy
arrays.  Every function below names the C routine it wraps; the page passages
each routine follows are cited in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zero1_oracle.c")
# ORACLE_LIB loads another build of the same source (the mutation test points
# it at builds with planted mistakes, to show that the pins catch them)
_BUILT = os.path.join(_HERE, "liboracle.so")
_LIB_PATH = os.environ.get("ORACLE_LIB") or _BUILT

GCC_FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
             "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]

NORM_BLOCK = 65536


def build() -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = _BUILT + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _BUILT)
    return _BUILT


_lib = None


class Scalars(ctypes.Structure):
    _fields_ = [("b1", ctypes.c_float), ("b2", ctypes.c_float),
                ("a1", ctypes.c_float), ("a2", ctypes.c_float),
                ("eps", ctypes.c_float), ("sigma", ctypes.c_float),
                ("delta", ctypes.c_float)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, f64, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [f32]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = f32
        L.oracle_f32_to_bf16_array.argtypes = [P, P, i64]
        L.oracle_f32_to_bf16_array.restype = None
        L.oracle_fp_env_ok.argtypes = []
        L.oracle_fp_env_ok.restype = i32
        L.oracle_shard_reduce.argtypes = [P, i32, i64, i32, P]
        L.oracle_shard_reduce.restype = None
        L.oracle_sumsq.argtypes = [P, i64, f64]
        L.oracle_sumsq.restype = f64
        L.oracle_global_norm.argtypes = [P, i32]
        L.oracle_global_norm.restype = f64
        L.oracle_clip_coef.argtypes = [f64, f64, ctypes.POINTER(f32)]
        L.oracle_clip_coef.restype = i32
        L.oracle_adamw_scalars.argtypes = [f64, f64, f64, f64, f64, i64, ctypes.POINTER(Scalars)]
        L.oracle_adamw_scalars.restype = None
        L.oracle_adamw.argtypes = [P, P, P, P, P, i64, ctypes.POINTER(Scalars), i32, f32]
        L.oracle_adamw.restype = None
        L.oracle_adamw_bf16mv.argtypes = [P, P, P, P, P, i64, ctypes.POINTER(Scalars), i32, f32]
        L.oracle_adamw_bf16mv.restype = None
        L.oracle_adamw_decay_first.argtypes = [P, P, P, P, i64, ctypes.POINTER(Scalars)]
        L.oracle_adamw_decay_first.restype = None
        L.oracle_step.argtypes = [P, i32, i64, i32, P, P, P, i32, P,
                                  f64, f64, f64, f64, f64, f64, i64,
                                  P, i32, i32, P, P]
        L.oracle_step.restype = i32
        L.oracle_step_v.argtypes = L.oracle_step.argtypes + [ctypes.c_uint]
        L.oracle_step_v.restype = i32
        L.oracle_clip_coef_eps.argtypes = [f64, f64, ctypes.POINTER(f32)]
        L.oracle_clip_coef_eps.restype = i32
        L.oracle_round_to_bf16.argtypes = [P, i64]
        L.oracle_round_to_bf16.restype = None
        L.oracle_zero_bytes_per_gpu.argtypes = [f64, f64, f64, i32]
        L.oracle_zero_bytes_per_gpu.restype = f64
        L.oracle_threads.argtypes = [i32]
        L.oracle_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


def _ptr_array(arrays) -> ctypes.Array:
    arr = (ctypes.c_void_p * len(arrays))()
    for k, a in enumerate(arrays):
        arr[k] = _ptr(a)
    return arr


# ---------------------------------------------------------------- formats
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of fp32 values (oracle_f32_to_bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def fp_env_ok() -> bool:
    return bool(lib().oracle_fp_env_ok())


# ---------------------------------------------------------------- steps
def shard_reduce(grads, average: bool = True) -> np.ndarray:
    """O1 (oracle_shard_reduce): fp32 sum of W bf16 slices in rank order, then / W."""
    grads = [np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    n = grads[0].size
    assert all(g.size == n for g in grads)
    out = np.empty(n, dtype=np.float32)
    keep = _ptr_array(grads)
    lib().oracle_shard_reduce(ctypes.cast(keep, ctypes.c_void_p), len(grads), n,
                              int(average), _ptr(out))
    return out


def sumsq(g: np.ndarray, total_in: float = 0.0) -> float:
    """O2 (oracle_sumsq): fixed-block fp64 sum of squares."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    return float(lib().oracle_sumsq(_ptr(g), g.size, float(total_in)))


def global_norm(rank_sumsq) -> float:
    a = np.ascontiguousarray(rank_sumsq, dtype=np.float64)
    return float(lib().oracle_global_norm(_ptr(a), a.size))


def clip_coef(norm: float, max_norm: float):
    """O3 (oracle_clip_coef): returns (clip_flag, fp32 coefficient)."""
    c = ctypes.c_float()
    flag = lib().oracle_clip_coef(float(norm), float(max_norm), ctypes.byref(c))
    return bool(flag), np.float32(c.value)


def clip_coef_eps(norm: float, max_norm: float):
    """Torch-convention clip (oracle_clip_coef_eps): returns (clip_flag, fp32 coefficient)."""
    c = ctypes.c_float()
    flag = lib().oracle_clip_coef_eps(float(norm), float(max_norm), ctypes.byref(c))
    return bool(flag), np.float32(c.value)


def round_to_bf16(g: np.ndarray) -> np.ndarray:
    """Copy of g rounded to bf16 and widened (oracle_round_to_bf16)."""
    out = np.ascontiguousarray(g, dtype=np.float32).copy()
    lib().oracle_round_to_bf16(_ptr(out), out.size)
    return out


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, t) -> Scalars:
    """O4 (oracle_adamw_scalars)."""
    s = Scalars()
    lib().oracle_adamw_scalars(lr, beta1, beta2, eps, weight_decay, int(t), ctypes.byref(s))
    return s


def adamw(g, master, m, v, param_bf16, scalars: Scalars, clip: bool, coef) -> None:
    """O5-O7 in place (oracle_adamw or oracle_adamw_bf16mv, chosen by m's dtype)."""
    n = g.size
    for a in (master, m, v, param_bf16):
        assert a.size == n and a.flags["C_CONTIGUOUS"]
    g = np.ascontiguousarray(g, dtype=np.float32)
    if m.dtype == np.uint16:
        lib().oracle_adamw_bf16mv(_ptr(g), _ptr(master), _ptr(m), _ptr(v), _ptr(param_bf16),
                                  n, ctypes.byref(scalars), int(clip), float(coef))
    else:
        assert m.dtype == np.float32 and v.dtype == np.float32
        lib().oracle_adamw(_ptr(g), _ptr(master), _ptr(m), _ptr(v), _ptr(param_bf16),
                           n, ctypes.byref(scalars), int(clip), float(coef))


def adamw_decay_first(g, master, m, v, scalars: Scalars) -> None:
    lib().oracle_adamw_decay_first(_ptr(g), _ptr(master), _ptr(m), _ptr(v), g.size,
                                   ctypes.byref(scalars))


class StepInfo:
    __slots__ = ("norm", "coef", "clip", "sumsq")

    def __init__(self, info):
        self.norm = float(info[0])
        self.coef = np.float32(info[1])
        self.clip = bool(info[2])
        self.sumsq = float(info[3])


DECAY_FIRST = 1
CLIP_EPS = 2
G_BF16 = 4


def step(grads, master, m, v, param_bf16, hp, rank_sumsq, my_rank, average=True, variant=0) -> StepInfo:
    """One rank's whole step on a flat shard (oracle_step), in place.

    grads: list of W uint16 arrays (this rank's slice of each replica);
    master fp32; m, v fp32 or uint16 (bf16 moments); param_bf16 uint16;
    hp: dict with lr, beta1, beta2, eps, weight_decay, max_norm, step;
    rank_sumsq: float64 array of all ranks' partials (entry my_rank is written).
    variant: DECAY_FIRST | CLIP_EPS | G_BF16 compatibility variants (0: the pages' step).
    """
    grads = [np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    n = master.size
    assert all(g.size == n for g in grads)
    assert rank_sumsq.dtype == np.float64 and rank_sumsq.flags["C_CONTIGUOUS"]
    mv_bf16 = m.dtype == np.uint16
    scratch = np.empty(n, dtype=np.float32)
    info = np.zeros(4, dtype=np.float64)
    keep = _ptr_array(grads)
    rc = lib().oracle_step_v(ctypes.cast(keep, ctypes.c_void_p), len(grads), n, int(average),
                             _ptr(master), _ptr(m), _ptr(v), int(mv_bf16), _ptr(param_bf16),
                             hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"],
                             hp["max_norm"], int(hp["step"]), _ptr(rank_sumsq), rank_sumsq.size,
                             int(my_rank), _ptr(scratch), _ptr(info), int(variant))
    if rc != 0:
        raise RuntimeError("oracle: the CPU flushes subnormals (FTZ/DAZ set)")
    return StepInfo(info)


def zero_bytes_per_gpu(psi, K, n_d, stage) -> float:
    return float(lib().oracle_zero_bytes_per_gpu(float(psi), float(K), float(n_d), int(stage)))


def threads(n: int = 0) -> int:
    """Set the OpenMP thread count of the oracle's loops (n > 0) and return
    the count in effect (oracle_threads; no arithmetic)."""
    return int(lib().oracle_threads(int(n)))
