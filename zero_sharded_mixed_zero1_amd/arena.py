"""One rank's optimizer arrays inside one device allocation, laid out by
zero1_arena_plan: the update's streams (g or gradient slice 0, master, m, v,
the bf16 parameters) far apart, which HBM serves faster on MI355X than one
allocation per array.  This module allocates the arena and hands out typed
views of its arrays; the offsets all come from the library's planner.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .binding import MV_BF16, ArenaLayout, arena_plan

ALIGN = 2 << 20   # the planner's offsets assume a 2 MiB-aligned base


@dataclass
class Arena:
    storage: object            # the one uint8 allocation (the views keep it alive)
    layout: ArenaLayout        # byte offsets from the aligned base
    base: int                  # offset of that base inside `storage`
    ws: object                 # uint8 [layout.ws_bytes]: the step's workspace
    master: object             # float32 [shard_len]
    m: object                  # float32 [shard_len], or int16 holding bf16 with MV_BF16
    v: object                  # likewise
    params: object             # int16 [param_elems]: the flat bf16 parameter buffer
    grads: list = field(default_factory=list)   # W x int16 [grad_elems]: the gradient buffers


def arena_tensors(shard_len: int, W: int, grad_elems: int, grad_offset: int, param_elems: int,
                  param_offset: int, flags: int = 0, device=None, capacity: int | None = None,
                  reserve: int = 8 << 30) -> Arena:
    """Allocate one arena for a rank's step and return views of its arrays.

    The arguments are zero1_arena_plan's: shard_len elements in the shard, W
    gradient buffers of grad_elems bf16 elements with the shard at grad_offset,
    a parameter buffer of param_elems bf16 elements with the shard at
    param_offset, flags MV_BF16 and the design (STORE_G, RECOMPUTE_G, or
    neither for the one zero1_mta_step picks: pass the same flags to the step).
    capacity: the largest arena to allocate; by default the device's free
    memory less `reserve` bytes.  The views are uninitialised.
    """
    import torch

    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if capacity is None:
        if dev.type != "cuda":
            raise ValueError("capacity must be given for a device other than a GPU")
        free, _ = torch.cuda.mem_get_info(dev)
        capacity = max(0, free - reserve - ALIGN)
    L = arena_plan(shard_len, W, grad_elems, grad_offset, param_elems, param_offset, flags, capacity)
    storage = torch.empty(L.total_bytes + ALIGN, dtype=torch.uint8, device=dev)
    base = (-storage.data_ptr()) % ALIGN

    def view(off, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return storage[base + off:base + off + nbytes].view(dt)

    mvdt = torch.int16 if flags & MV_BF16 else torch.float32
    return Arena(storage, L, base, view(L.ws, L.ws_bytes, torch.uint8), view(L.master, shard_len, torch.float32),
                 view(L.m, shard_len, mvdt), view(L.v, shard_len, mvdt), view(L.params, param_elems, torch.int16),
                 [view(L.grads[w], grad_elems, torch.int16) for w in range(W)])
