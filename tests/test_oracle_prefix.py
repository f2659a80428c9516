"""Pins of the prefix-cache oracle (Primer chapter 8, section 8.3: hash the
prompt in block-sized pieces, map cached blocks, prefill and register the
rest).  The hash is FNV-1a 64, checked on the test vectors published with
its definition; the cache on closed cases."""

import pytest

from oracle.allocator import Pool, PoolError
from oracle.prefix_cache import BLOCK, PrefixCache, block_keys, fnv1a64


def test_fnv1a64_published_vectors():
    # FNV reference test vectors for the 64-bit FNV-1a variant
    assert fnv1a64(b"") == 0xcbf29ce484222325
    assert fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert fnv1a64(b"foobar") == 0x85944171f73967e8


def test_keys_chain_over_the_prefix():
    a = list(range(100))
    b = a[:40] + [999] + a[41:]                 # token 40 (block 2) differs
    ka, kb = block_keys(a), block_keys(b)
    assert len(ka) == 6 and len(block_keys(a[:47])) == 2   # full blocks only
    assert ka[:2] == kb[:2] and all(x != y for x, y in zip(ka[2:], kb[2:]))
    # the same block after a different prefix gets another key
    c = [7] * 16 + a[16:32]
    assert block_keys(c)[1] != ka[1]


def _pool(n=40):
    return Pool(n, body_free_order=list(range(n)))


def _prefill(pool, ids, sid=None):
    if sid is None:
        sid = pool.seq_create()
    pool.seq_reserve(sid, len(ids) - pool.seq_len(sid))
    return sid


def test_register_then_lookup_maps_every_full_block():
    pool = _pool()
    cache = PrefixCache(pool)
    ids = list(range(70))                       # 4 full blocks + 6 tokens
    s0 = _prefill(pool, ids)
    assert cache.register(s0, ids) == 4
    t0 = pool.seq_table(s0)
    assert [pool.refcount(b) for b in t0] == [2, 2, 2, 2, 1]
    s1, n = cache.lookup(ids + [5, 6])
    assert n == 64 and pool.seq_table(s1) == t0[:4] and pool.seq_len(s1) == 64
    assert [pool.refcount(b) for b in t0[:4]] == [3] * 4
    assert cache.stats() == (4, 4, 4)
    # the next write opens a new block: nothing shared is written
    pool.seq_reserve(s1, 8)
    assert pool.seq_table(s1)[4] not in t0 and pool.copies == []


def test_lookup_stops_at_the_first_divergent_block():
    pool = _pool()
    cache = PrefixCache(pool)
    ids = list(range(64))
    cache.register(_prefill(pool, ids), ids)
    other = ids[:32] + [-1] + ids[33:]
    sid, n = cache.lookup(other)
    assert n == 32 and len(pool.seq_table(sid)) == 2


def test_eviction_is_lru_among_leaves_held_by_the_cache_only():
    pool = _pool(20)
    cache = PrefixCache(pool)
    a = list(range(48))
    b = list(range(100, 132))
    sa = _prefill(pool, a)
    cache.register(sa, a)
    sb = _prefill(pool, b)
    cache.register(sb, b)
    ta, tb = pool.seq_table(sa), pool.seq_table(sb)
    assert cache.evict(10) == 0                 # every block still held by a sequence
    pool.seq_release(sa)
    pool.seq_release(sb)
    free0 = pool.num_free(0)
    cache.lookup(a[:16])                        # a's first block is used again
    assert cache.evict(1) == 1                  # the LRU leaf: a's last block
    assert ta[2] in pool.free_stack(0)[:1] and pool.num_free(0) == free0 + 1
    assert cache.evict(1) == 1                  # then a's second block (now a leaf)
    assert ta[1] in pool.free_stack(0)[:1]
    assert cache.evict(10) == 2                 # b's blocks, leaf first; a's first is in use
    assert pool.free_stack(0)[:2] == [tb[0], tb[1]]
    assert cache.stats()[0] == 1


def test_window_pools_are_refused():
    pool = Pool(8, 4, 1, window_tokens=32)
    with pytest.raises(PoolError) as e:
        PrefixCache(pool).lookup(list(range(32)))
    assert e.value.code == "UNSUPPORTED"


def test_a_planted_unchained_key_is_caught():
    """Mutation check: keys of each block alone (no chain) would let a block
    match after a different prefix; the chained keys do not."""
    def unchained(ids):
        return [fnv1a64(b"".join((t % (1 << 32)).to_bytes(4, "little") for t in ids[i:i + BLOCK]))
                for i in range(0, len(ids) - BLOCK + 1, BLOCK)]
    x = [1] * 16 + list(range(16))
    y = [2] * 16 + list(range(16))
    assert unchained(x)[1] == unchained(y)[1]
    assert block_keys(x)[1] != block_keys(y)[1]
