"""One data-parallel rank's ZeRO-1 optimizer step on MI355X (gfx950).

Thin Python binding over libzero1.so (C ABI in include/zero1.h).  This module
only marshals arguments: every step of the path (reduce, norm, clip, AdamW,
bf16 copy) runs in the library's HIP kernels.  There is no CPU fallback: if the
library is missing, importing the binding functions raises.
"""
from .binding import (  # noqa: F401
    Zero1Error, HParams, NormInfo, Piece, Plan, ArenaRequest, ArenaLayout, StepScalars,
    SUM_ONLY, MV_BF16, RECOMPUTE_G, STORE_G, DECAY_FIRST, CLIP_EPS, G_BF16, MAX_W, STATIC_MAX_G_ELEMS,
    abi_version, last_error, shard_range, workspace_bytes,
    shard_reduce, grad_norm, adamw_step,
    mta_table_bytes, mta_plan, mta_workspace_bytes, mta_reduce, mta_update, mta_design, mta_step,
    mta_step_static, mta_reduce_range, partials_sum,
    arena_plan, step_scalars_derive, time_next_launch,
    lib, lib_path,
)
from .layout import shard_pieces  # noqa: F401
from .arena import Arena, arena_tensors  # noqa: F401
