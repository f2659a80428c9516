"""Pins of the oracle's local FP16 window (CPU).

What the pages fix (8GB page, section 4, "The Hybrid Solution"): the first 8
tokens (attention sinks) and the most recent 128 tokens stay FP16 in
dedicated high-precision blocks; the middle body is INT4 per head and per
group of 64 dims.  The oracle's reading (per-block precision, blocks leave
the window whole, ``seq_settle`` moves them) is pinned here by closed forms,
invariants on every reachable state of small op logs, and the decode-step
schedule of migrations.
"""

import itertools
import random

import numpy as np
import pytest

from oracle.allocator import BODY, SINK, Pool, PoolError

W = 128


def _pool(nb=4096, ns=64, window=W, seed=0):
    r = np.random.default_rng(seed)
    return Pool(nb, ns, 1, body_free_order=r.permutation(nb), sink_free_order=r.permutation(ns),
                window_tokens=window)


def _fp16_tokens(p, sid):
    """Tokens of the sequence held in FP16 blocks."""
    L = p.seq_len(sid)
    return sum(min(16, L - 16 * j) for j, b in enumerate(p.seq_table(sid)) if p.arena_of(b) == SINK)


def _shape_ok(p, sid):
    """Table = sink blocks, then body blocks, then FP16 blocks."""
    arenas = [p.arena_of(b) for b in p.seq_table(sid)]
    k = p.sink_per_seq
    if any(a != SINK for a in arenas[:k]):
        return False
    rest = arenas[k:]
    first_sink = next((i for i, a in enumerate(rest) if a == SINK), len(rest))
    return all(a == SINK for a in rest[first_sink:])


@pytest.mark.parametrize("L", [1, 16, 128, 143, 144, 145, 160, 1000, 65536])
def test_prefill_routes_blocks_by_final_position(L):
    """A prefill of L tokens takes the blocks out of the window straight from
    the body: FP16 holds the sink block plus a tail of W..W+15 tokens (all of
    them when L <= W + 16), and settling moves nothing."""
    p = _pool()
    s = p.seq_create()
    p.seq_reserve(s, L)
    assert p.seq_settle(s) == 0 and _shape_ok(p, s)
    n_out = max(0, (L - W) // 16)
    body = max(0, n_out - 1)
    assert sum(p.arena_of(b) == BODY for b in p.seq_table(s)) == body
    tail = L - 16 * max(n_out, 1)
    if L > 16 + W:
        assert W <= tail <= W + 15
    assert _fp16_tokens(p, s) == L - 16 * body


def test_decode_steps_migrate_one_block_every_16_tokens():
    p = _pool()
    s = p.seq_create()
    p.seq_reserve(s, 1000)
    p.seq_settle(s)
    moves = []
    for step in range(80):
        p.seq_reserve(s, 1)
        moves.append(p.seq_settle(s))
        assert _shape_ok(p, s)
        assert W <= _fp16_tokens(p, s) - 16 <= W + 15   # sink block + the window tail
    # (1000 + k - 128) // 16 grows by one exactly when 1000 + k - 128 hits a multiple of 16
    want = [((1000 + k + 1 - W) // 16) - ((1000 + k - W) // 16) for k in range(80)]
    assert moves == want and sum(moves) == 5


def test_migrations_pop_lifo_in_logical_order():
    p = Pool(8, 8, 1, body_free_order=[5, 2, 7, 0, 1, 3, 4, 6],
             sink_free_order=list(range(8)), window_tokens=32)
    s = p.seq_create()
    p.seq_reserve(s, 64)            # blocks: sink, body(j=1 out: 16*2 <= 32), fp16 x2
    assert [p.arena_of(b) for b in p.seq_table(s)] == [SINK, BODY, SINK, SINK]
    p.seq_reserve(s, 32)            # now 96 tokens: j = 2, 3 out of the window
    fp16_before = [p.seq_table(s)[j] for j in (2, 3)]
    assert p.seq_settle(s) == 2
    assert p.migrations[-2:] == [(fp16_before[0], 2), (fp16_before[1], 7)]
    # the FP16 blocks went back to the sink stack, last freed on top
    assert p.free_stack(SINK)[:2] == [fp16_before[1], fp16_before[0]]


def test_settle_is_all_or_nothing():
    q = Pool(1, 8, 1, window_tokens=64)
    t = q.seq_create()
    for _ in range(8):
        q.seq_reserve(t, 16)        # every block starts in the window (FP16)
    state = (q.seq_table(t), q.free_stack(BODY), q.free_stack(SINK))
    with pytest.raises(PoolError):
        q.seq_settle(t)             # 3 blocks left the window, the body has 1
    assert (q.seq_table(t), q.free_stack(BODY), q.free_stack(SINK)) == state


def _random_logs(seed, n=40):
    rnd = random.Random(seed)
    ops = []
    nseq = 0
    for _ in range(n):
        k = rnd.randrange(6)
        if k == 0 or nseq == 0:
            ops.append(("create",))
            nseq += 1
        elif k == 1:
            ops.append(("reserve", rnd.randrange(nseq), rnd.choice([1, 1, 3, 17, 40])))
        elif k == 2:
            ops.append(("settle", rnd.randrange(nseq)))
        elif k == 3:
            ops.append(("fork", rnd.randrange(nseq)))
            nseq += 1
        elif k == 4:
            ops.append(("truncate", rnd.randrange(nseq), rnd.randrange(0, 60)))
        else:
            ops.append(("release", rnd.randrange(nseq)))
    return ops


@pytest.mark.parametrize("seed", range(40))
def test_invariants_on_random_logs(seed):
    """Every reachable state: tables have the sink/body/FP16 shape, refcounts
    equal the number of table uses, free stacks and used blocks partition each
    arena, and after a settle no FP16 block of a sequence is out of its window."""
    from oracle.allocator import replay
    p = Pool(40, 24, 1, body_free_order=np.random.default_rng(seed).permutation(40),
             window_tokens=32)
    for op in _random_logs(seed):
        replay(p, [op])
        uses = {}
        for sid in p.seqs:
            assert _shape_ok(p, sid)
            for b in p.seq_table(sid):
                uses[b] = uses.get(b, 0) + 1
        for b in range(64):
            assert p.ref[b] == uses.get(b, 0)
        assert sorted(p.free_stack(BODY) + [b for b in uses if b < 40]) == list(range(40))
        if op[0] == "settle" and op[1] in p.seqs:
            t = p.seq_table(op[1])
            n_out = p.n_out(p.seq_len(op[1]))
            assert all(p.arena_of(t[j]) == BODY for j in range(1, min(n_out, len(t))))
