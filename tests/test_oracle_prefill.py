"""Pins of the chunked-prefill oracle (8GB page, section 5, "Notice two
critical details", item 1 "Chunked Prefill"): slicing a prompt into chunks changes no result, so the chunked
evaluation (per-query prefix loops, the verify step's operation) must equal
causal attention written as one masked score matrix, for every chunk size;
plus closed forms that hold whatever the chunking."""

import numpy as np
import pytest

from oracle import attention as AT


def _inputs(P, hq=4, hkv=2, D=16, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((P, hq, D)), r.standard_normal((P, hkv, D)),
            r.standard_normal((P, hkv, D)))


@pytest.mark.parametrize("chunk", [1, 3, 16, 37, 64, 100])
def test_chunked_equals_one_pass_causal(chunk):
    q, K, V = _inputs(100)
    full = AT.causal_attention(q, K, V, 0.25)
    got = AT.prefill_chunks(q, K, V, 0.25, chunk)
    assert np.allclose(got, full, rtol=0, atol=1e-12)


def test_first_query_sees_only_the_first_token():
    q, K, V = _inputs(20, seed=1)
    out = AT.prefill_chunks(q, K, V, 0.3, 8)
    for h in range(4):
        assert np.array_equal(out[0, h], V[0, h // 2])


def test_last_query_is_the_decode_of_the_whole_prompt():
    q, K, V = _inputs(50, seed=2)
    out = AT.prefill_chunks(q, K, V, 0.2, 16)
    assert np.allclose(out[-1], AT.attention_one(q[-1], K, V, 0.2), rtol=0, atol=1e-13)


def test_equal_keys_give_prefix_means():
    """All keys equal: every visible token has the same score, so query i's
    output is the mean of V[0..i] (closed form)."""
    q, K, V = _inputs(30, seed=3)
    K[:] = K[0]
    out = AT.prefill_chunks(q, K, V, 0.5, 7)
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, 31)[:, None, None]
    for h in range(4):
        assert np.allclose(out[:, h], prefix_mean[:, h // 2], rtol=0, atol=1e-12)


def test_a_planted_future_leak_is_caught():
    """Mutation check on the pin: letting queries see the whole chunk (no
    causal mask inside it) must break the equality."""
    q, K, V = _inputs(32, seed=4)
    full = AT.causal_attention(q, K, V, 0.25)
    leaky = np.concatenate([np.stack([AT.attention_one(q[i], K[:16 * (i // 16 + 1)], V[:16 * (i // 16 + 1)], 0.25)
                                      for i in range(s, s + 16)]) for s in (0, 16)])
    assert not np.allclose(leaky, full, atol=1e-6)
