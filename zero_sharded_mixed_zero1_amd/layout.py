"""Host-side layout of a ragged tensor list under ZeRO-1 sharding.

The parameter list is flattened in list order into one vector of N elements;
rank r of W owns the contiguous flat range [r*S, (r+1)*S) with S = ceil(N/W)
(the reduce-scatter convention that rank i receives block i: page "并行训练",
section "卡和卡怎么说话：集合通信").  A shard boundary can fall inside a
tensor, so a rank's shard is a list of PIECES, each a contiguous part of one
tensor.  This module only computes that bookkeeping; it does no arithmetic on
parameter values.
"""
from __future__ import annotations


def shard_pieces(numels, begin: int, end: int):
    """Pieces of the flat range [begin, end) over tensors with sizes `numels`.

    Returns a list of (tensor_index, offset_in_tensor, shard_offset, numel),
    in flat order; shard_offset is the position inside [begin, end).
    """
    out = []
    base = 0
    for idx, n in enumerate(numels):
        lo, hi = max(base, begin), min(base + n, end)
        if lo < hi:
            out.append((idx, lo - base, lo - begin, hi - lo))
        base += n
        if base >= end:
            break
    return out
