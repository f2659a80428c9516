"""Seeded synthetic workloads for paged decode attention.

This module only draws random inputs and writes down workload recipes
(shapes, lengths, free orders, the order of allocator operations).  It holds
none of the method's arithmetic: no allocation policy, no quantization, no
attention.  Both the library's tests/bench and the CPU oracle take their inputs
from here.

Recipe (one ``numpy.random.default_rng`` stream per purpose, keyed by
``(seed, tag, index)``, so any one array can be drawn without the others):

* tag 0: sequence lengths, then the free-order permutation of the body arena;
* tag 1: K of sequence b (``float32`` N(0,1), shape ``[L_b][Hkv][D]``);
* tag 2: V of sequence b;
* tag 3: Q (``[B][Hq][D]``);
* tag 4: the outlier channels of the mixed-precision workload;
* tag 5: the free-order permutation of the sink arena;
* tag 6: K of appended decode tokens (index = step), tag 106: their V;
* tag 7: the queries of a speculative verify step (index = queries per
  sequence, shape ``[B][n_query][Hq][D]``).

A ``reserve`` of n tokens on a sequence of length L writes tokens
``[L, L+n)`` of that sequence's logical content (``Workload.seq_tokens``); a
forked child's content starts with its parent's tokens, which it shares.

Lengths and pool sizes follow the workloads the pages use as examples: a
Llama-3-8B-shaped layer with 32 query heads, 8 KV heads and head_dim 128
(8GB page, section 2), 16-token blocks (8GB page, section 3), a 64k context
(8GB page, section 4), sink blocks in FP16 with an INT4/FP8 body (same
section) and a shared system prompt (8GB page, section 3, copy-on-write).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


def rng(seed, tag, index=0):
    return np.random.default_rng([int(seed), int(tag), int(index)])


@dataclass
class Workload:
    name: str
    seed: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_dtype: str                 # "f32" | "f16" | "bf16" | "int4" | "fp8"
    q_dtype: str                  # "f32" | "f16" | "bf16"
    in_dtype: str                 # dtype of K/V handed to the append call
    num_blocks: int
    body_free_order: np.ndarray
    ops: list                     # allocator op log, see oracle.allocator.replay
    decode_seqs: list             # sequence ids that form the decode batch
    token_src: dict               # seq id -> list of (tag, index, count) K/V sources
    group_size: int = 0
    num_sink_blocks: int = 0
    sink_blocks_per_seq: int = 0
    sink_free_order: np.ndarray | None = None
    outlier_channels: np.ndarray | None = None
    outlier_scale: float = 10.0
    window_tokens: int = 0
    block_size: int = BLOCK       # tokens per pool block (8 and 32: raw 16-bit, D 128)
    extra: dict = field(default_factory=dict)
    softmax_scale: float | None = None  # None: 1 / sqrt(head_dim)

    @property
    def batch(self):
        return len(self.decode_seqs)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim) if self.softmax_scale is None else self.softmax_scale

    def q(self):
        return rng(self.seed, 3).standard_normal(
            (self.batch, self.n_q_heads, self.head_dim), dtype=np.float32)

    def q_verify(self, n_query):
        """Queries of a verify step over the last n_query cached tokens."""
        return rng(self.seed, 7, n_query).standard_normal(
            (self.batch, n_query, self.n_q_heads, self.head_dim), dtype=np.float32)

    def q_chunk(self, k, n):
        """Queries of prefill chunk k (n tokens per sequence)."""
        return rng(self.seed, 8, k).standard_normal(
            (self.batch, n, self.n_q_heads, self.head_dim), dtype=np.float32)

    def kv_chunk(self, tag, index, count):
        """K and V (float32 [count][Hkv][D]) of one source chunk."""
        shape = (count, self.n_kv_heads, self.head_dim)
        k = rng(self.seed, 1 if tag == 1 else tag, index).standard_normal(shape, dtype=np.float32)
        v = rng(self.seed, 2 if tag == 1 else tag + 100, index).standard_normal(shape, dtype=np.float32)
        if self.outlier_channels is not None:
            h, d = np.divmod(self.outlier_channels, self.head_dim)
            k[:, h, d] *= self.outlier_scale
            v[:, h, d] *= self.outlier_scale
        return k, v

    def seq_tokens(self, sid):
        """All K/V tokens a sequence writes, in order (float32)."""
        ks, vs = [], []
        for tag, index, count in self.token_src[sid]:
            k, v = self.kv_chunk(tag, index, count)
            ks.append(k)
            vs.append(v)
        shape = (0, self.n_kv_heads, self.head_dim)
        if not ks:
            return np.zeros(shape, np.float32), np.zeros(shape, np.float32)
        return np.concatenate(ks), np.concatenate(vs)


def _pool_size(blocks_needed):
    return int(math.ceil(1.1 * blocks_needed))


def _prefill_ops(lengths):
    ops = [("create",) for _ in lengths]
    ops += [("reserve", b, int(L)) for b, L in enumerate(lengths)]
    return ops


def tiny(seed=1):
    """3 sequences of 25, 47 and 12 tokens (3-minute page's worked example),
    64-block pool in seeded random order, 4 q / 4 kv heads, head_dim 64, fp32."""
    lengths = [25, 47, 12]
    perm = rng(seed, 0).permutation(64)
    return Workload("tiny", seed, 4, 4, 64, "f32", "f32", "f32", 64, perm,
                    _prefill_ops(lengths), [0, 1, 2],
                    {b: [(1, b, L)] for b, L in enumerate(lengths)},
                    extra={"lengths": lengths})


def llama3_8b(seed=2, batch=64, min_len=512, max_len=4096, block_size=BLOCK):
    """Llama-3-8B-shaped decode layer: 32 q / 8 kv heads, head_dim 128, bf16,
    lengths uniform in [min_len, max_len], pool = blocks needed + 10 %.
    block_size 8 or 32: the same batch in a pool of that block size (the
    block-size trade of the 3-minute page, "Compartilhamento e compromissos")."""
    r = rng(seed, 0)
    lengths = [int(x) for x in r.integers(min_len, max_len + 1, size=batch)]
    n = _pool_size(sum(-(-L // block_size) for L in lengths))
    perm = r.permutation(n)
    name = "llama3-8b" + ("" if block_size == BLOCK else f"-bs{block_size}")
    return Workload(name, seed, 32, 8, 128, "bf16", "bf16", "bf16", n, perm,
                    _prefill_ops(lengths), list(range(batch)),
                    {b: [(1, b, L)] for b, L in enumerate(lengths)},
                    block_size=block_size, extra={"lengths": lengths})


def long_context(seed=3, batch=4, length=65536):
    """batch sequences of ``length`` tokens each, 32 q / 8 kv heads, bf16."""
    lengths = [length] * batch
    n = _pool_size(batch * (-(-length // BLOCK)))
    perm = rng(seed, 0).permutation(n)
    return Workload("long-context", seed, 32, 8, 128, "bf16", "bf16", "bf16", n, perm,
                    _prefill_ops(lengths), list(range(batch)),
                    {b: [(1, b, length)] for b in range(batch)},
                    extra={"lengths": lengths})


def mixed_precision(seed=4, kv="int4", length=65536, steps=64, group=128,
                    n_kv_heads=8, head_dim=128, n_q_heads=32, window=0):
    """One sequence of ``length`` fp16 tokens, then ``steps`` single-token
    appends.  Logical block 0 (16 sink tokens) lives in a one-block FP16 sink
    arena, the body is INT4 (groups of ``group``) or FP8.  1 % of the
    (head, dim) channels are scaled x10 in K and V for every token.  With
    ``window`` > 0 the FP16 arena also holds the blocks of the last
    ``window`` tokens, and every reserve is followed by a settle."""
    body_blocks = -(-(length + steps - BLOCK) // BLOCK)
    n = _pool_size(body_blocks)
    perm = rng(seed, 0).permutation(n)
    n_out = int(round(0.01 * n_kv_heads * head_dim))
    outl = np.sort(rng(seed, 4).choice(n_kv_heads * head_dim, size=n_out, replace=False))
    settle = [("settle", 0)] if window else []
    ops = [("create",), ("reserve", 0, length)] + settle
    for _ in range(steps):
        ops += [("reserve", 0, 1)] + settle
    src = [(1, 0, length)] + [(6, s, 1) for s in range(steps)]
    n_sink = 1 + (-(-window // BLOCK) + 2 if window else 0)
    name = f"mixed-{kv}" + (f"-w{window}-g{group}" if window else "")
    return Workload(name, seed, n_q_heads, n_kv_heads, head_dim, kv, "f16", "f16",
                    n, perm, ops, [0], {0: src}, group_size=group if kv == "int4" else 0,
                    num_sink_blocks=n_sink, sink_blocks_per_seq=1,
                    sink_free_order=rng(seed, 5).permutation(n_sink) if window else np.arange(1),
                    outlier_channels=outl, window_tokens=window,
                    extra={"lengths": [length + steps], "steps": steps, "prefill": length})


def window_batch(lengths, steps=0, window=128, group=64, kv="int4", n_q_heads=32, n_kv_heads=8,
                 head_dim=128, seed=12, settle=True, chunk=1):
    """Sequences of the given lengths with a one-block FP16 sink and a local
    FP16 window of ``window`` tokens, then ``steps`` steps that each add
    ``chunk`` tokens per sequence (1: decode steps; more: verify steps or
    prefill chunks), each followed by a settle unless ``settle`` is False:
    then the blocks that leave the window stay FP16, and a chunk of several
    blocks leaves the table with FP16 runs between body runs.  INT4 groups
    of ``group`` or FP8 body, 1 % outlier channels x10."""
    lengths = [int(L) for L in lengths]
    B = len(lengths)
    grow = steps * chunk
    body = sum(max(0, -(-(L + grow) // BLOCK) - 1) for L in lengths)
    n = max(1, _pool_size(body))
    n_sink = B * (1 + -(-window // BLOCK) + 2 + (0 if settle else steps * (-(-window // BLOCK) + 1)
                                                  + -(-grow // BLOCK)))
    ops = []
    src = {}
    for b, L in enumerate(lengths):
        ops += [("create",), ("reserve", b, L), ("settle", b)]
        src[b] = [(1, b, L)]
    for s in range(steps):
        for b in range(B):
            ops += [("reserve", b, chunk)] + ([("settle", b)] if settle else [])
            src[b].append((6, s * 4096 + b, chunk))
    n_o = max(1, int(round(0.01 * n_kv_heads * head_dim)))
    outl = np.sort(rng(seed, 4).choice(n_kv_heads * head_dim, size=n_o, replace=False))
    return Workload(f"window-{kv}-w{window}" + ("" if settle else "-lag"), seed, n_q_heads, n_kv_heads, head_dim, kv, "f16", "f16",
                    n, rng(seed, 0).permutation(n), ops, list(range(B)), src,
                    group_size=group if kv == "int4" else 0, num_sink_blocks=n_sink,
                    sink_blocks_per_seq=1, sink_free_order=rng(seed, 5).permutation(n_sink),
                    outlier_channels=outl, window_tokens=window,
                    extra={"lengths": [L + grow for L in lengths], "steps": steps})


def chunked_prefill(seed=9, lengths=(4096, 4096, 4096, 4096), chunk=512, n_q_heads=32, n_kv_heads=8,
                    head_dim=128, dt="bf16"):
    """Prompts prefilled in chunks of `chunk` tokens (8GB page, section 5,
    "Notice two critical details", item 1 "Chunked Prefill"):
    round k reserves (and writes) every unfinished prompt's next chunk, so
    the sequences' blocks interleave in the pool as a chunk scheduler would
    leave them.  Chunk k's queries: q_chunk(k, n)."""
    lengths = [int(L) for L in lengths]
    B = len(lengths)
    n = _pool_size(sum(-(-L // BLOCK) for L in lengths))
    ops = [("create",) for _ in range(B)]
    for s0 in range(0, max(lengths + [0]), chunk):
        for b, L in enumerate(lengths):
            if s0 < L:
                ops.append(("reserve", b, min(chunk, L - s0)))
    return Workload("prefill-chunk", seed, n_q_heads, n_kv_heads, head_dim, dt, dt, dt, n,
                    rng(seed, 0).permutation(n), ops, list(range(B)),
                    {b: [(1, b, L)] for b, L in enumerate(lengths)},
                    extra={"lengths": lengths, "chunk": chunk})


def shared_prefix(seed=5, prefix=2000, n_children=32, max_suffix=512):
    """An owner sequence holds a ``prefix``-token prompt; ``n_children`` forks
    each add a suffix of uniform length in [0, max_suffix].  64 q / 8 kv
    heads, head_dim 128, bf16.  Pool size is an upper bound on the blocks
    needed (prefix + suffix blocks + one possible clone each) + 10 %."""
    r = rng(seed, 0)
    suffix = [int(x) for x in r.integers(0, max_suffix + 1, size=n_children)]
    bound = -(-prefix // BLOCK) + sum(-(-u // BLOCK) + 1 for u in suffix)
    n = _pool_size(bound)
    perm = r.permutation(n)
    ops = [("create",), ("reserve", 0, prefix)]
    ops += [("fork", 0) for _ in range(n_children)]
    ops += [("reserve", c + 1, u) for c, u in enumerate(suffix)]
    src = {0: [(1, 0, prefix)]}
    for c, u in enumerate(suffix):
        src[c + 1] = [(1, 0, prefix), (1, c + 1, u)]
    return Workload(f"shared-prefix-{prefix}", seed, 64, 8, 128, "bf16", "bf16", "bf16",
                    n, perm, ops, list(range(1, n_children + 1)), src,
                    extra={"lengths": [prefix + u for u in suffix], "prefix": prefix,
                           "suffix": suffix})


def from_lengths(lengths, n_q_heads=32, n_kv_heads=8, head_dim=128, kv_dtype="bf16", seed=11,
                 name="custom", group=0, sink=False, outliers=False, block_size=BLOCK):
    """Sequences of the given lengths (prefilled sequence-major), pool of the
    blocks needed + 10 % in a seeded random order.  For a quantized body,
    ``sink=True`` puts logical block 0 in a FP16 sink arena."""
    lengths = [int(L) for L in lengths]
    qdt = kv_dtype if kv_dtype in ("f32", "f16", "bf16") else "f16"
    n_sink = len(lengths) if sink else 0
    body = sum(max(0, -(-L // block_size) - (1 if sink else 0)) for L in lengths)
    n = max(1, _pool_size(body))
    perm = rng(seed, 0).permutation(n)
    outl = None
    if outliers:
        n_out = max(1, int(round(0.01 * n_kv_heads * head_dim)))
        outl = np.sort(rng(seed, 4).choice(n_kv_heads * head_dim, size=n_out, replace=False))
    return Workload(name, seed, n_q_heads, n_kv_heads, head_dim, kv_dtype, qdt, qdt, n, perm,
                    _prefill_ops(lengths), list(range(len(lengths))),
                    {b: [(1, b, L)] for b, L in enumerate(lengths)},
                    group_size=group, num_sink_blocks=n_sink,
                    sink_blocks_per_seq=1 if sink else 0,
                    sink_free_order=rng(seed, 5).permutation(n_sink) if sink else None,
                    outlier_channels=outl, block_size=block_size, extra={"lengths": lengths})


def by_name(name, **kw):
    table = {
        "tiny": tiny,
        "llama3-8b": llama3_8b,
        "long-context": long_context,
        "mixed-int4": lambda **k: mixed_precision(kv="int4", **k),
        "mixed-fp8": lambda **k: mixed_precision(kv="fp8", **k),
        "shared-prefix": shared_prefix,
        "shared-prefix-partial": lambda **k: shared_prefix(prefix=1992, **k),
        "spec-verify": llama3_8b,   # the same batch, scored by a verify step
        # the mixed-precision sequence scored by a verify step (gamma = 5)
        "spec-verify-int4": lambda **k: mixed_precision(kv="int4", **k),
        "spec-verify-window": lambda **k: mixed_precision(kv="int4", group=64, window=128, **k),
        "llama3-8b-bs8": lambda **k: llama3_8b(block_size=8, **k),
        "llama3-8b-bs32": lambda **k: llama3_8b(block_size=32, **k),
        # the pages' own scheme: FP16 sink block and last-128-token window, INT4 g = 64
        "mixed-window": lambda **k: mixed_precision(kv="int4", group=64, window=128, **k),
        # 4 prompts of 4,096 tokens in 512-token chunks; the bench times the last chunk
        "prefill-chunk": chunked_prefill,
    }
    return table[name](**kw)
