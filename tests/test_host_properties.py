"""Property tests (hypothesis) of the host-side bookkeeping, no GPU:

* zero1_shard_range: W shards of S = ceil(N/W) cover [0, N) exactly once, in
  rank order (rank i owns block i: "并行训练", "卡和卡怎么说话：集合通信");
* shard_pieces: a shard of a ragged tensor list is cut into pieces that tile
  it in flat order, each inside one tensor;
* zero1_arena_plan: no two arrays overlap, every buffer starts on a 2 MiB
  boundary, the spaced arrays' shard ranges sit exactly one spacing apart,
  and the arena fits the capacity."""
from __future__ import annotations

from hypothesis import given, settings
from hypothesis import strategies as st

import zero_sharded_mixed_zero1_amd as z
from synth.workloads import shard_range as py_shard_range

MiB2 = 2 << 20


@settings(max_examples=300, deadline=None)
@given(N=st.integers(0, 10**12), W=st.integers(1, 128))
def test_shard_range_covers_exactly_once(N, W):
    pos = 0
    for r in range(W):
        b, n = z.shard_range(N, W, r)
        assert (b, b + n) == py_shard_range(N, W, r)
        assert b == min(pos, N) and n >= 0
        pos = b + n
        assert n <= -(-N // W)
    assert pos == N


@settings(max_examples=300, deadline=None)
@given(numels=st.lists(st.integers(1, 5000), min_size=1, max_size=40), data=st.data())
def test_shard_pieces_tile_the_range(numels, data):
    N = sum(numels)
    begin = data.draw(st.integers(0, N))
    end = data.draw(st.integers(begin, N))
    ps = z.shard_pieces(numels, begin, end)
    pos = 0
    offs = [0]
    for n in numels:
        offs.append(offs[-1] + n)
    last = -1
    for ti, off, so, n in ps:
        assert ti > last and n > 0 and so == pos
        assert 0 <= off and off + n <= numels[ti]
        assert offs[ti] + off == begin + so
        pos += n
        last = ti
    assert pos == end - begin


@settings(max_examples=300, deadline=None)
@given(S=st.integers(1, 2 * 10**9), W=st.integers(1, 128), full=st.booleans(),
       flags=st.sampled_from([0, z.STORE_G, z.RECOMPUTE_G, z.MV_BF16, z.STORE_G | z.MV_BF16]),
       cap_gib=st.integers(1, 400), data=st.data())
def test_arena_plan_invariants(S, W, full, flags, cap_gib, data):
    ge, go = (S * W, data.draw(st.integers(0, S * (W - 1)))) if full else (S, 0)
    pe = S + data.draw(st.integers(0, 10**6))
    po = data.draw(st.integers(0, pe - S))
    cap = cap_gib << 30
    try:
        L = z.arena_plan(S, W, ge, go, pe, po, flags, capacity=cap)
    except z.Zero1Error as e:
        assert e.name == "ZERO1_EINVAL" and "packed layout" in e.message
        return
    assert L.total_bytes <= cap
    mvb = 2 if flags & z.MV_BF16 else 4
    spans = [(L.master, 4 * S), (L.m, mvb * S), (L.v, mvb * S), (L.params, 2 * pe), (L.ws, L.ws_bytes)]
    spans += [(L.grads[w], 2 * ge) for w in range(W)]
    for off, _ in spans:
        assert off % 2 == 0
    for off in (L.master, L.m, L.v, L.params + 2 * po):
        assert off % MiB2 == 0
    assert L.m - L.master == L.spacing and L.v - L.m == L.spacing and L.params + 2 * po - L.v == L.spacing
    spans.sort()
    for (a0, n0), (a1, _) in zip(spans, spans[1:]):
        assert a0 + n0 <= a1
    assert spans[-1][0] + spans[-1][1] <= L.total_bytes
