"""Oracle accounting: KV bytes, slots, waste.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* KV bytes = 2 * n_layers * n_kv_heads * d_head * s_seq * b * sizeof(dtype)
  (8GB page, section 2, "First-Principles Math"; the printed formula is
  garbled, the variable list under it fixes the factors).
* INT4 with groups of g values: g/2 bytes of codes plus 4 bytes of fp16
  (scale, zero) per group (8GB page, section 4, INT4 byte count).
* FP8: one byte per element; the page's 64 KiB/token ignores the scale.
* A paged sequence uses its length rounded up to the block size; a contiguous
  one reserves max_context (3-minute page, "A analogia com memoria virtual").
"""

from __future__ import annotations


def kv_bytes(n_layers, n_kv_heads, d_head, s_seq, b, sizeof):
    return 2 * n_layers * n_kv_heads * d_head * s_seq * b * sizeof


def int4_bytes_per_token(n_layers, n_kv_heads, d_head, group):
    elems = 2 * n_layers * n_kv_heads * d_head
    return elems // group * (group // 2 + 4)


def fp8_bytes_per_token(n_layers, n_kv_heads, d_head, with_scale=False, scale_bytes=2):
    per_head = d_head + (scale_bytes if with_scale else 0)
    return 2 * n_layers * n_kv_heads * per_head


def blocks_for(length, block=16):
    return (length + block - 1) // block


def paged_slots(lengths, block=16):
    return sum(block * blocks_for(L, block) for L in lengths)


def contiguous_slots(n_seqs, max_context):
    return n_seqs * max_context


def tail_waste(length, block=16):
    return block * blocks_for(length, block) - length
