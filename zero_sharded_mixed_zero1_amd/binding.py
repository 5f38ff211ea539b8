"""ctypes binding of libzero1.so: the same names as the C ABI (include/zero1.h).

Argument marshalling only.  Device buffers may be given as torch CUDA tensors
(their data_ptr is passed) or as raw integer device addresses; `stream` is a
torch.cuda.Stream, a raw hipStream_t integer, or None for torch's current
stream.  Every call raises Zero1Error on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ZERO1_LIB points the binding at another build of the same library (for
# instance one built with other compile-time launch constants)
lib_path = os.environ.get("ZERO1_LIB") or os.path.join(HERE, "libzero1.so")

SUM_ONLY = 0x1
MV_BF16 = 0x2
RECOMPUTE_G = 0x4
STORE_G = 0x8
DECAY_FIRST = 0x20
CLIP_EPS = 0x40
G_BF16 = 0x80
MAX_W = 128
STATIC_MAX_G_ELEMS = 16777216
# the layout of the structures below and the signatures set in lib(); a
# library that reports another ZERO1_ABI_VERSION is refused at load time
ABI_VERSION = 4

P = ctypes.c_void_p
i64 = ctypes.c_int64
i32 = ctypes.c_int
u32 = ctypes.c_uint32
szt = ctypes.c_size_t


class Zero1Error(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name
        self.message = message


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("max_norm", ctypes.c_double), ("step", i64), ("device_scalars", P)]


class StepScalars(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("one_minus_beta1", ctypes.c_float), ("one_minus_beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("step_size", ctypes.c_float), ("decay", ctypes.c_float),
                ("reserved", ctypes.c_float), ("max_norm", ctypes.c_double)]


class NormInfo(ctypes.Structure):
    _fields_ = [("sumsq_total", ctypes.c_double), ("norm", ctypes.c_double),
                ("clip_coef", ctypes.c_float), ("clip", ctypes.c_int32),
                ("nonfinite", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Piece(ctypes.Structure):
    _fields_ = [("numel", i64), ("shard_offset", i64), ("param_bf16", P), ("master", P),
                ("m", P), ("v", P)]


class Plan(ctypes.Structure):
    _fields_ = [("table", P), ("shard_len", i64), ("n_pieces", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("chunk_elems", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("aligned", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ArenaRequest(ctypes.Structure):
    _fields_ = [("shard_len", i64), ("W", i32), ("grad_elems", i64), ("grad_offset", i64),
                ("param_elems", i64), ("param_offset", i64), ("flags", ctypes.c_uint32),
                ("capacity", ctypes.c_size_t)]


class ArenaLayout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("spacing", ctypes.c_size_t),
                ("ws", ctypes.c_size_t), ("ws_bytes", ctypes.c_size_t),
                ("master", ctypes.c_size_t), ("m", ctypes.c_size_t), ("v", ctypes.c_size_t),
                ("params", ctypes.c_size_t), ("grads", ctypes.c_size_t * 128)]


_lib = None


def lib():
    """The loaded libzero1.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is not built: run __graft_entry__.build() "
                              "(the HIP library is the only implementation)")
        # PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7, which its
        # libraries load by the file name libamdhip64.so).  Loading torch first
        # lets libzero1's libamdhip64.so.7 resolve to that same copy; loaded the
        # other way round, the process would hold two HIP runtimes, and the
        # second to initialise finds no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(lib_path)
        L.zero1_abi_version.argtypes = []
        L.zero1_abi_version.restype = i32
        if L.zero1_abi_version() != ABI_VERSION:
            raise ImportError(f"{lib_path} has ABI version {L.zero1_abi_version()}, this binding expects "
                              f"{ABI_VERSION}: rebuild the library with __graft_entry__.build()")
        L.zero1_last_error.argtypes = []
        L.zero1_last_error.restype = ctypes.c_char_p
        L.zero1_status_string.argtypes = [i32]
        L.zero1_status_string.restype = ctypes.c_char_p
        L.zero1_shard_range.argtypes = [i64, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.zero1_shard_range.restype = i32
        L.zero1_workspace_bytes.argtypes = [i64, i32, u32]
        L.zero1_workspace_bytes.restype = szt
        L.zero1_shard_reduce.argtypes = [P, i32, i64, i64, u32, P, P, P, szt, P]
        L.zero1_shard_reduce.restype = i32
        L.zero1_grad_norm.argtypes = [P, i64, P, P, szt, P]
        L.zero1_grad_norm.restype = i32
        L.zero1_adamw_step.argtypes = [P, P, i32, i64, i64, P, P, P, P, ctypes.POINTER(HParams),
                                       P, i32, u32, P, P]
        L.zero1_adamw_step.restype = i32
        L.zero1_mta_table_bytes.argtypes = [ctypes.POINTER(Piece), i32]
        L.zero1_mta_table_bytes.restype = szt
        L.zero1_mta_plan.argtypes = [ctypes.POINTER(Piece), i32, u32, P, szt, ctypes.POINTER(Plan)]
        L.zero1_mta_plan.restype = i32
        L.zero1_mta_workspace_bytes.argtypes = [ctypes.POINTER(Plan), i32, u32]
        L.zero1_mta_workspace_bytes.restype = szt
        L.zero1_mta_reduce.argtypes = [P, i32, i64, ctypes.POINTER(Plan), P, u32, P, szt, P]
        L.zero1_mta_reduce.restype = i32
        L.zero1_mta_update.argtypes = [P, i32, i64, ctypes.POINTER(Plan), ctypes.POINTER(HParams),
                                       P, i32, u32, P, P, szt, P]
        L.zero1_mta_update.restype = i32
        L.zero1_mta_reduce_range.argtypes = [P, i32, ctypes.POINTER(Plan), i64, i64, P, u32, P, szt, P]
        L.zero1_mta_reduce_range.restype = i32
        L.zero1_partials_sum.argtypes = [P, i32, P, P]
        L.zero1_partials_sum.restype = i32
        L.zero1_mta_design.argtypes = [P, i32, i64, ctypes.POINTER(Plan), u32]
        L.zero1_mta_design.restype = i32
        L.zero1_mta_step.argtypes = [P, i32, i64, ctypes.POINTER(Plan), ctypes.POINTER(HParams),
                                     P, i32, i32, u32, P, P, szt, P]
        L.zero1_mta_step.restype = i32
        L.zero1_mta_step_static.argtypes = [P, i32, i64, ctypes.POINTER(Plan), ctypes.POINTER(HParams),
                                            P, i32, i32, u32, P, P]
        L.zero1_mta_step_static.restype = i32
        L.zero1_step_scalars_derive.argtypes = [ctypes.POINTER(HParams), ctypes.POINTER(StepScalars)]
        L.zero1_step_scalars_derive.restype = i32
        L.zero1_arena_plan.argtypes = [ctypes.POINTER(ArenaRequest), ctypes.POINTER(ArenaLayout)]
        L.zero1_arena_plan.restype = i32
        L.zero1_time_next_launch.argtypes = [P, P]
        L.zero1_time_next_launch.restype = i32
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling
def _check(st: int):
    if st != 0:
        L = lib()
        raise Zero1Error(st, L.zero1_status_string(st).decode(), L.zero1_last_error().decode())


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not getattr(x, "is_cuda", True):
            raise ValueError("device buffer expected, got a CPU tensor")
        return x.data_ptr()
    raise TypeError(f"cannot take a device address of {type(x)}")


def _nbytes(x) -> int:
    if hasattr(x, "untyped_storage"):
        return x.numel() * x.element_size()
    raise TypeError("workspace size must be given with a raw address")


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptrs(grads):
    arr = (ctypes.c_void_p * len(grads))()
    for k, g in enumerate(grads):
        arr[k] = _addr(g)
    return arr


def _ws(ws, ws_bytes):
    if ws is None:
        return 0, 0
    return _addr(ws), (ws_bytes if ws_bytes is not None else _nbytes(ws))


def _hp(hp) -> HParams:
    """From an HParams, or a dict with lr, beta1, beta2, eps, weight_decay,
    max_norm, step and optionally device_scalars (a device address or tensor
    holding a StepScalars; the other keys are then ignored)."""
    if isinstance(hp, HParams):
        return hp
    dev = hp.get("device_scalars")
    if dev is not None:
        return HParams(0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0, _addr(dev))
    return HParams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"],
                   hp["max_norm"], int(hp["step"]), None)


def step_scalars_derive(hp) -> StepScalars:
    """The per-step scalars the step calls derive from hp (zero1_step_scalars_derive)."""
    out = StepScalars()
    h = _hp(hp)
    _check(lib().zero1_step_scalars_derive(ctypes.byref(h), ctypes.byref(out)))
    return out


# ------------------------------------------------------------------ ABI
def abi_version() -> int:
    return lib().zero1_abi_version()


def last_error() -> str:
    return lib().zero1_last_error().decode()


def shard_range(n_total: int, W: int, rank: int):
    b, n = i64(), i64()
    _check(lib().zero1_shard_range(n_total, W, rank, ctypes.byref(b), ctypes.byref(n)))
    return b.value, n.value


def workspace_bytes(length: int, W: int, flags: int = 0) -> int:
    return lib().zero1_workspace_bytes(length, W, flags)


def shard_reduce(grads, begin: int, length: int, g_out=None, sumsq_out=None, flags: int = 0,
                 ws=None, ws_bytes=None, stream=None):
    arr = _ptrs(grads)
    w, wb = _ws(ws, ws_bytes)
    _check(lib().zero1_shard_reduce(ctypes.cast(arr, P), len(grads), begin, length, flags,
                                    _addr(g_out), _addr(sumsq_out), w, wb, _stream(stream)))


def grad_norm(g, length: int, sumsq_out, ws=None, ws_bytes=None, stream=None):
    w, wb = _ws(ws, ws_bytes)
    _check(lib().zero1_grad_norm(_addr(g), length, _addr(sumsq_out), w, wb, _stream(stream)))


def adamw_step(g, grads, begin: int, length: int, master, m, v, param_bf16, hp, rank_sumsq,
               n_ranks: int, flags: int = 0, info_out=None, stream=None):
    grads = list(grads) if grads is not None else []
    arr = _ptrs(grads) if grads else None
    h = _hp(hp)
    _check(lib().zero1_adamw_step(_addr(g), ctypes.cast(arr, P) if arr is not None else None,
                                  len(grads), begin, length, _addr(master), _addr(m), _addr(v),
                                  _addr(param_bf16), ctypes.byref(h), _addr(rank_sumsq), n_ranks,
                                  flags, _addr(info_out), _stream(stream)))


def _pieces(pieces):
    if isinstance(pieces, ctypes.Array):
        return pieces
    arr = (Piece * len(pieces))()
    for k, p in enumerate(pieces):
        if isinstance(p, Piece):
            arr[k] = p
        else:
            numel, off, param, master, m, v = p
            arr[k] = Piece(numel, off, _addr(param), _addr(master), _addr(m), _addr(v))
    return arr


def mta_table_bytes(pieces) -> int:
    arr = _pieces(pieces)
    return lib().zero1_mta_table_bytes(arr, len(arr))


def mta_plan(pieces, table, table_bytes=None, flags: int = 0) -> Plan:
    """pieces: Piece structs or tuples (numel, shard_offset, param_bf16, master, m, v)."""
    arr = _pieces(pieces)
    plan = Plan()
    t, tb = _ws(table, table_bytes)
    _check(lib().zero1_mta_plan(arr, len(arr), flags, t, tb, ctypes.byref(plan)))
    return plan


def mta_workspace_bytes(plan: Plan, W: int, flags: int = 0) -> int:
    return lib().zero1_mta_workspace_bytes(ctypes.byref(plan), W, flags)


def mta_reduce(grads, begin: int, plan: Plan, sumsq_out, flags: int = 0, ws=None, ws_bytes=None,
               stream=None):
    arr = _ptrs(grads)
    w, wb = _ws(ws, ws_bytes)
    _check(lib().zero1_mta_reduce(ctypes.cast(arr, P), len(grads), begin, ctypes.byref(plan),
                                  _addr(sumsq_out), flags, w, wb, _stream(stream)))


def mta_update(grads, begin: int, plan: Plan, hp, rank_sumsq, n_ranks: int, flags: int = 0,
               info_out=None, ws=None, ws_bytes=None, stream=None):
    arr = _ptrs(grads)
    w, wb = _ws(ws, ws_bytes)
    h = _hp(hp)
    _check(lib().zero1_mta_update(ctypes.cast(arr, P), len(grads), begin, ctypes.byref(plan),
                                  ctypes.byref(h), _addr(rank_sumsq), n_ranks, flags,
                                  _addr(info_out), w, wb, _stream(stream)))


def mta_reduce_range(grads, plan: Plan, lo: int, hi: int, sumsq_out, flags: int = STORE_G, ws=None,
                     ws_bytes=None, stream=None):
    """grads[w] addresses replica w's gradient of shard element lo."""
    arr = _ptrs(grads)
    w, wb = _ws(ws, ws_bytes)
    _check(lib().zero1_mta_reduce_range(ctypes.cast(arr, P), len(grads), ctypes.byref(plan), lo, hi,
                                        _addr(sumsq_out), flags, w, wb, _stream(stream)))


def partials_sum(parts, n: int, sum_out, stream=None):
    _check(lib().zero1_partials_sum(_addr(parts), n, _addr(sum_out), _stream(stream)))


def mta_design(grads, begin: int, plan: Plan, flags: int = 0) -> int:
    """The design flag (STORE_G or RECOMPUTE_G) mta_step would run; 0 if none."""
    arr = _ptrs(grads)
    return lib().zero1_mta_design(ctypes.cast(arr, P), len(grads), begin, ctypes.byref(plan), flags)


def mta_step(grads, begin: int, plan: Plan, hp, rank_sumsq, n_ranks: int, my_rank: int,
             flags: int = 0, info_out=None, ws=None, ws_bytes=None, stream=None):
    arr = _ptrs(grads)
    w, wb = _ws(ws, ws_bytes)
    h = _hp(hp)
    _check(lib().zero1_mta_step(ctypes.cast(arr, P), len(grads), begin, ctypes.byref(plan),
                                ctypes.byref(h), _addr(rank_sumsq), n_ranks, my_rank, flags,
                                _addr(info_out), w, wb, _stream(stream)))


def mta_step_static(grads, begin: int, plan: Plan, hp, rank_sumsq, n_ranks: int, my_rank: int,
                    flags: int = 0, info_out=None, stream=None):
    """zero1_mta_step with the workspace in the library's static device array."""
    arr = _ptrs(grads)
    h = _hp(hp)
    _check(lib().zero1_mta_step_static(ctypes.cast(arr, P), len(grads), begin, ctypes.byref(plan),
                                       ctypes.byref(h), _addr(rank_sumsq), n_ranks, my_rank, flags,
                                       _addr(info_out), _stream(stream)))


def arena_plan(shard_len: int, W: int, grad_elems: int, grad_offset: int, param_elems: int,
               param_offset: int, flags: int = 0, capacity: int = 1 << 62) -> ArenaLayout:
    """Byte offsets of one rank's arrays inside one arena (zero1_arena_plan)."""
    req = ArenaRequest(shard_len, W, grad_elems, grad_offset, param_elems, param_offset, flags, capacity)
    out = ArenaLayout()
    _check(lib().zero1_arena_plan(ctypes.byref(req), ctypes.byref(out)))
    return out


def _event(e) -> int:
    """A hipEvent_t from a raw integer handle or a torch.cuda.Event (torch
    creates its event at the first record, so an unrecorded one is recorded
    once on torch's current stream to bring it into existence)."""
    if e is None:
        return 0
    if isinstance(e, int):
        return e
    if not e.cuda_event:
        e.record()
    return e.cuda_event


def time_next_launch(start=None, stop=None):
    """The first kernel of this thread's next step call records start/stop
    (zero1_time_next_launch): start.elapsed_time(stop) is that kernel's own
    duration.  Events need enable_timing=True."""
    _check(lib().zero1_time_next_launch(_event(start), _event(stop)))
