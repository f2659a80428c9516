"""Oracle reading of the pool's byte layout, written from the specification in
``include/pa.h`` (section "Pool memory layout").  It shares no code with the
library: it is an independent implementation of that text, used to read back
what the GPU stored and to lay out expected data.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix the shape of the packed INT4 store as
``[num_blocks, n_kv_heads, block_size, head_dim // 2]`` bytes with per-token,
per-group fp16 scale and zero arrays of shape
``[num_blocks, n_kv_heads, block_size, head_dim // group_size]``
(8GB page, section 7, "Register-Level INT4 Dequantization in PagedAttention").
The library keeps that outer order (block, head, then a 16-token slab) and
fixes its own order *inside* each slab; the index functions below spell out
that order for every array.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16
DT_F32, DT_F16, DT_BF16, DT_INT4, DT_FP8 = 0, 1, 2, 3, 4
ELEM = {DT_F32: 4, DT_F16: 2, DT_BF16: 2}


def _td(D, bs=BLOCK):
    t = np.arange(bs)[:, None]
    d = np.arange(D)[None, :]
    return np.broadcast_to(t, (bs, D)), np.broadcast_to(d, (bs, D))


def _sub_slabs(bs):
    """Tokens per sub-slab (S) and sub-slabs per block: a 32-token block is
    two 16-token slabs back to back, an 8-token block one slab of S = 8."""
    S = 8 if bs == 8 else 16
    return S, bs // S


def raw_k_index(D, bs=BLOCK):
    """Element index of K[t][d] inside a raw block of bs tokens: sub-slab
    t // S, then [d/8][t % S][d%8] inside it."""
    S, _ = _sub_slabs(bs)
    t, d = _td(D, bs)
    return (t // S) * S * D + ((d // 8) * S + t % S) * 8 + d % 8


def raw_v_index(D, bs=BLOCK):
    """Element index of V[t][d] inside a raw block of bs tokens (sub-slab
    t // S of S tokens, then the rule inside it).

    With NT = D/16: row r = d / NT, tile T = d % NT, token group g = (t%S)/4,
    i = t % 4, unit u = T / 2, parity p = T % 2:
    index = ((u*(S/4)*16 + g*16 + r)*2 + p)*4 + i  (u*64 at S = 16).
    """
    S, _ = _sub_slabs(bs)
    t, d = _td(D, bs)
    nt = D // 16
    r, T = d // nt, d % nt
    ts = t % S
    g, i = ts // 4, ts % 4
    u, p = T // 2, T % 2
    return (t // S) * S * D + ((u * (S // 4) * 16 + g * 16 + r) * 2 + p) * 4 + i


def int4_k_byte(D):
    """(byte index, nibble shift) of K code [t][d] inside an INT4 K slab.

    k = d/2, step kk = k/16, lane group g = (k%16)/4, b = k%4:
    byte = ((g*16 + t)*(D/32) + kk)*4 + b; even d in the low nibble.
    """
    t, d = _td(D)
    k = d // 2
    kk, g, b = k // 16, (k % 16) // 4, k % 4
    return ((g * BLOCK + t) * (D // 32) + kk) * 4 + b, (d % 2) * 4


def int4_v_byte(D):
    """(byte index, nibble shift) of V code [t][d] inside an INT4 V slab.

    NT = D/16, r = d / NT, j = (d % NT)/2, g = t/4, i = t%4:
    byte = ((g*16 + r)*(NT/2) + j)*4 + i; even d in the low nibble.
    """
    t, d = _td(D)
    nt = D // 16
    r, j = d // nt, (d % nt) // 2
    g, i = t // 4, t % 4
    return ((g * 16 + r) * (nt // 2) + j) * 4 + i, (d % 2) * 4


def fp8_k_byte(D):
    """Byte index of K code [t][d] inside an FP8 K slab.

    kk = d/32, s = kk/2, h = kk%2, g = (d%32)/8, j = d%8:
    byte = ((s*4 + g)*16 + t)*16 + h*8 + j.
    """
    t, d = _td(D)
    kk = d // 32
    s, h, g, j = kk // 2, kk % 2, (d % 32) // 8, d % 8
    return ((s * 4 + g) * BLOCK + t) * 16 + h * 8 + j


def fp8_v_byte(D):
    """Byte index of V code [t][d] inside an FP8 V slab.

    NT = D/16, r = d / NT, T = d % NT, u = T/4, T4 = T%4, g = t/4, i = t%4:
    byte = ((u*64 + g*16 + r)*4 + T4)*4 + i.
    """
    t, d = _td(D)
    nt = D // 16
    r, T = d // nt, d % nt
    u, T4 = T // 4, T % 4
    g, i = t // 4, t % 4
    return ((u * 64 + g * 16 + r) * 4 + T4) * 4 + i


# ---- whole-pool array placement ----------------------------------------------
def _align(x, a=256):
    return (x + a - 1) // a * a


def pool_arrays(kv_dtype, n_kv_heads, head_dim, group_size, num_blocks, num_sink_blocks,
                block_size=BLOCK):
    """Ordered list of (name, byte offset, bytes per (block, head) slab, arena
    block count) for every array in the pool, and the total byte size.
    block_size other than 16 only for raw pools (the others are fixed at 16)."""
    H, D, N, S = n_kv_heads, head_dim, num_blocks, num_sink_blocks
    items = []
    if kv_dtype in ELEM:
        e = ELEM[kv_dtype]
        items += [("K", block_size * D * e, N), ("V", block_size * D * e, N)]
    elif kv_dtype == DT_INT4:
        ng = D // group_size
        items += [("KC", BLOCK * D // 2, N), ("VC", BLOCK * D // 2, N),
                  ("KS", BLOCK * ng * 2, N), ("KZ", BLOCK * ng * 2, N),
                  ("VS", BLOCK * ng * 2, N), ("VZ", BLOCK * ng * 2, N)]
    elif kv_dtype == DT_FP8:
        items += [("KC", BLOCK * D, N), ("VC", BLOCK * D, N),
                  ("KS", BLOCK * 2, N), ("VS", BLOCK * 2, N)]
    else:
        raise ValueError(kv_dtype)
    if S > 0:
        items += [("SK", BLOCK * D * 2, S), ("SV", BLOCK * D * 2, S)]
    out, off = [], 0
    for name, slab, nblk in items:
        off = _align(off)
        out.append((name, off, slab, nblk))
        off += slab * H * nblk
    return out, _align(off)


def array_view(pool_bytes, arrays, name, n_kv_heads, dtype):
    """View one array as [blocks][heads][slab elements] of ``dtype``."""
    for nm, off, slab, nblk in arrays:
        if nm == name:
            raw = np.asarray(pool_bytes, dtype=np.uint8)[off:off + slab * n_kv_heads * nblk]
            return raw.view(dtype).reshape(nblk, n_kv_heads, -1)
    raise KeyError(name)


# ---- logical rebuild (one sequence, one kv head) -------------------------------
def gather_raw(slabs, ids, head, D, which, bs=BLOCK):
    """Logical [len(ids)*bs][D] values of K or V from raw slabs of bs tokens."""
    idx = raw_k_index(D, bs) if which == "K" else raw_v_index(D, bs)
    return np.concatenate([slabs[b, head][idx] for b in ids], axis=0)


def gather_int4_codes(slabs, ids, head, D, which):
    byte, sh = int4_k_byte(D) if which == "K" else int4_v_byte(D)
    return np.concatenate([(slabs[b, head][byte] >> sh) & 0xF for b in ids], axis=0)


def gather_fp8_codes(slabs, ids, head, D, which):
    byte = fp8_k_byte(D) if which == "K" else fp8_v_byte(D)
    return np.concatenate([slabs[b, head][byte] for b in ids], axis=0)


def gather_rows(slabs, ids, head):
    """Per-token metadata (scales, zeros): slab is [16][groups] row-major."""
    return np.concatenate([slabs[b, head].reshape(BLOCK, -1) for b in ids], axis=0)
