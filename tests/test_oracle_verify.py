"""Pins of the oracle's speculative verify step (CPU).

What the pages fix (8GB page, section 6): the target model scores the
gamma + 1 new tokens in one pass; the section 5 flowchart rolls the rejected
tail back.  The oracle's reading (query i sees the cache up to its own token)
is pinned here against things other than itself:

* a library routine: torch's scaled_dot_product_attention in float64 with an
  explicit boolean mask ``t <= L - nq + i`` per query row;
* special cases: one query is plain decode of the whole cache; a query whose
  position precedes the cache start has a zero row; a single visible token
  returns its V exactly; planted mistakes (off-by-one causal edge, the full
  cache for every query, queries in reversed order) fail the library pin;
* the rollback: reserving the step's tokens and truncating them again leaves
  the pool exactly as it was (LIFO: the blocks come back in order), also
  across a copy-on-write of a shared tail.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as AT
from oracle.allocator import Pool


def _sdpa_verify(q, K, V, scale):
    """q [nq][Hq][D], K/V [L][Hkv][D] -> [nq][Hq][D] through torch (float64)."""
    nq, hq, _ = q.shape
    L, hkv, _ = K.shape
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][nq][D]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    t = torch.arange(L)[None, :]
    i = torch.arange(nq)[:, None]
    mask = t <= (L - nq + i)                                        # [nq][L]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("nq,hq,hkv,L,D", [(6, 32, 8, 40, 16), (2, 4, 4, 2, 8), (6, 8, 2, 6, 8),
                                           (3, 6, 3, 17, 4), (1, 4, 2, 9, 8)])
def test_verify_vs_masked_sdpa(nq, hq, hkv, L, D):
    rnd = np.random.default_rng(nq * 100 + L)
    q = rnd.standard_normal((nq, hq, D))
    K = rnd.standard_normal((L, hkv, D)) * 3
    V = rnd.standard_normal((L, hkv, D))
    got = AT.verify_attention_one(q, K, V, 1 / math.sqrt(D))
    assert np.allclose(got, _sdpa_verify(q, K, V, 1 / math.sqrt(D)), rtol=0, atol=1e-12)


def test_verify_special_cases():
    rnd = np.random.default_rng(3)
    q = rnd.standard_normal((6, 4, 8))
    K = rnd.standard_normal((20, 2, 8))
    V = rnd.standard_normal((20, 2, 8))
    out = AT.verify_attention_one(q, K, V, 0.5)
    # the last query is the decode of the whole cache
    assert np.allclose(out[-1], AT.attention_one(q[-1], K, V, 0.5), rtol=0, atol=0)
    # a cache of 3 tokens and 6 queries: queries 0..2 precede it (zero rows),
    # query 3 sees token 0 only and returns its V exactly
    out = AT.verify_attention_one(q, K[:3], V[:3], 0.5)
    assert np.all(out[:3] == 0)
    assert np.array_equal(out[3], V[0][np.arange(4) // 2])


def test_verify_mutations_are_caught():
    rnd = np.random.default_rng(11)
    q = rnd.standard_normal((6, 8, 16))
    K = rnd.standard_normal((37, 2, 16)) * 3
    V = rnd.standard_normal((37, 2, 16))
    ref = _sdpa_verify(q, K, V, 0.25)

    def off_by_one(q, K, V, scale):  # query i sees one token fewer
        out = np.zeros(q.shape)
        for i in range(q.shape[0]):
            n = K.shape[0] - q.shape[0] + i
            if n > 0:
                out[i] = AT.attention_one(q[i], K[:n], V[:n], scale)
        return out

    def no_mask(q, K, V, scale):     # every query sees the whole cache
        return np.stack([AT.attention_one(q[i], K, V, scale) for i in range(q.shape[0])])

    def reversed_queries(q, K, V, scale):
        return AT.verify_attention_one(q[::-1], K, V, scale)[::-1]

    for bad in (off_by_one, no_mask, reversed_queries):
        assert not np.allclose(bad(q, K, V, 0.25), ref, atol=1e-6)


def _state(pool, seqs):
    return (pool.free_stack(0), [pool.refcount(i) for i in range(pool.n_body)],
            [pool.seq_table(s) for s in seqs], [pool.seq_len(s) for s in seqs])


@pytest.mark.parametrize("start,gamma,accepted", [(30, 5, 0), (30, 5, 3), (27, 5, 6), (32, 5, 2),
                                                  (1, 5, 1)])
def test_rollback_restores_the_pool(start, gamma, accepted):
    """Reserve the gamma + 1 tokens of a step, keep `accepted` of them,
    truncate the rest: the pool is the one a plain reserve of the accepted
    tokens gives; rejecting all of them restores the pool exactly."""
    perm = np.random.default_rng(start).permutation(24)
    a = Pool(24, body_free_order=perm)
    b = Pool(24, body_free_order=perm)
    for p in (a, b):
        s = p.seq_create()
        p.seq_reserve(s, start)
    before = _state(a, [0])
    a.seq_reserve(0, gamma + 1)
    a.seq_truncate(0, start + accepted)
    b.seq_reserve(0, accepted) if accepted else None
    assert _state(a, [0]) == _state(b, [0])
    if accepted == 0:
        assert _state(a, [0]) == before


def test_rollback_after_copy_on_write():
    """A fork writes its step into a shared partial tail: the tail is cloned
    first.  Rejecting the step keeps the clone (it holds the fork's copy of
    the tail tokens; truncation never re-shares); cutting into the tail
    returns the clone to the top of the free stack, and the parent's blocks
    keep their references throughout."""
    a = Pool(16, body_free_order=np.arange(16)[::-1].copy())
    p = a.seq_create()
    a.seq_reserve(p, 20)          # blocks 15 (full) and 14 (4 tokens)
    c = a.seq_fork(p)
    assert a.refcount(14) == 2
    a.seq_reserve(c, 6)           # clone of the shared tail, then the new tokens
    clone = a.seq_table(c)[1]
    assert clone not in (14, 15) and a.refcount(14) == 1 and a.refcount(clone) == 1
    a.seq_truncate(c, 20)         # all 6 rejected: same length, own tail copy
    assert a.seq_table(c) == [15, clone] and a.seq_len(c) == 20
    assert a.refcount(15) == 2 and a.refcount(14) == 1 and a.refcount(clone) == 1
    a.seq_truncate(c, 16)
    assert a.seq_table(c) == [15] and a.refcount(clone) == 0
    assert a.free_stack(0)[0] == clone  # next to be popped
    assert a.seq_table(p) == [15, 14] and a.seq_len(p) == 20
