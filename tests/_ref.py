"""Test-side glue between workloads and the oracle (CPU).

Builds, from a workload's seeded inputs and the oracle only, the values the
library must store and the outputs it must produce.  Nothing here calls the
library.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import attention as AT
from oracle import quant as QT
from oracle.allocator import Pool, replay

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def cast64(x, dt):
    """fp32 numpy -> stored dtype (torch's RNE cast) -> float64."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[dt]).to(torch.float64).numpy()


def oracle_pool(wl):
    """The oracle's pool after the workload's op log (tables, arenas)."""
    pool = Pool(wl.num_blocks, wl.num_sink_blocks, wl.sink_blocks_per_seq,
                body_free_order=wl.body_free_order, sink_free_order=wl.sink_free_order,
                window_tokens=wl.window_tokens, block_size=wl.block_size)
    replay(pool, wl.ops)
    return pool


def fp16_tokens(wl, pool, sid):
    """Per token of the sequence: True where its block is in the FP16 arena."""
    t = pool.seq_table(sid)
    return np.array([t[p // wl.block_size] >= wl.num_blocks for p in range(pool.seq_len(sid))],
                    dtype=bool)


def stored_values(wl, sid, fp16=None):
    """Float64 [L][Hkv][D] K and V the pool must hold for sequence sid, plus
    (for quantized bodies) the oracle's codes/scales/zeros of every token
    (the pool holds them for the tokens of body blocks).  ``fp16``: per-token
    mask of the FP16-arena tokens (default: the sink blocks)."""
    K, V = wl.seq_tokens(sid)
    if wl.kv_dtype in TORCH_DT:
        return cast64(K, wl.kv_dtype), cast64(V, wl.kv_dtype), None
    Kh = cast64(K, "f16").astype(np.float16)
    Vh = cast64(V, "f16").astype(np.float16)
    L = Kh.shape[0]
    if fp16 is None:
        fp16 = np.arange(L) < 16 * wl.sink_blocks_per_seq
    Kq, Vq = Kh.astype(np.float64), Vh.astype(np.float64)
    codes = {}
    if L == 0 or fp16.all():
        return Kq, Vq, {}
    body = ~fp16
    if wl.kv_dtype == "int4":
        for name, X, out in (("K", Kh, Kq), ("V", Vh, Vq)):
            q, s, z = QT.int4_quantize(X, wl.group_size)
            out[body] = QT.int4_dequant(q, s, z, wl.group_size)[body]
            codes[name], codes[name + "S"], codes[name + "Z"] = q, s, z
    else:
        for name, X, out in (("K", Kh, Kq), ("V", Vh, Vq)):
            c, s = QT.fp8_quantize(X)
            out[body] = QT.fp8_dequant(c, s)[body]
            codes[name], codes[name + "S"] = c, s
    return Kq, Vq, codes


def q_values(wl):
    return cast64(wl.q(), wl.q_dtype)


def expected(wl, seqs=None, pairs=None):
    """Oracle outputs [B][Hq][D] (float64); with ``pairs`` = list of (b, hq)
    only those rows are computed (others NaN)."""
    seqs = wl.decode_seqs if seqs is None else seqs
    q = q_values(wl)
    out = np.full((len(seqs), wl.n_q_heads, wl.head_dim), np.nan)
    want = None if pairs is None else {}
    if pairs is not None:
        for b, h in pairs:
            want.setdefault(b, []).append(h)
    pool = oracle_pool(wl) if wl.window_tokens else None
    for b, sid in enumerate(seqs):
        if want is not None and b not in want:
            continue
        K, V, _ = stored_values(wl, sid, fp16_tokens(wl, pool, sid) if pool else None)
        full = AT.attention_one(q[b], K, V, wl.scale)
        if want is None:
            out[b] = full
        else:
            for h in want[b]:
                out[b, h] = full[h]
    return out


def expected_verify(wl, n_query, seqs=None, rows=None):
    """Oracle verify-step outputs [B][n_query][Hq][D] (float64); with ``rows``
    = list of b only those sequences are computed (others NaN)."""
    seqs = wl.decode_seqs if seqs is None else seqs
    q = cast64(wl.q_verify(n_query), wl.q_dtype)
    out = np.full((len(seqs), n_query, wl.n_q_heads, wl.head_dim), np.nan)
    pool = oracle_pool(wl) if wl.window_tokens else None
    for b, sid in enumerate(seqs):
        if rows is not None and b not in rows:
            continue
        K, V, _ = stored_values(wl, sid, fp16_tokens(wl, pool, sid) if pool else None)
        out[b] = AT.verify_attention_one(q[b], K, V, wl.scale)
    return out


# (fraction bits, least normal exponent) of the output dtypes
_FMT = {"f32": (23, -126), "bf16": (7, -126), "f16": (10, -14)}


def round_to(x, out_dtype):
    """float64 values rounded to the nearest value of the output dtype, ties
    to even, exactly (x / ulp is exact: ulp is a power of two).  Values are
    assumed inside the dtype's range."""
    x = np.asarray(x, np.float64)
    mant, emin = _FMT[out_dtype]
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** (emin - mant)))), emin)
    ulp = 2.0 ** (e - mant)
    return np.round(x / ulp) * ulp          # numpy rounds halves to even


def bar(out_dtype):
    """Max |error| of the kernel's fp32 result against the oracle: 1e-5 for
    fp32 outputs, 2e-3 for bf16/fp16 (raw or quantized pools)."""
    return 1e-5 if out_dtype == "f32" else 2e-3


def assert_close(got, ref, out_dtype, what=""):
    """The output holds the kernel's fp32 result rounded once to out_dtype.
    It passes iff it is the rounding of some value within bar(out_dtype) of
    the oracle: rn(ref - bar) <= got <= rn(ref + bar) (rounding is monotone),
    so the only slack beyond the bar is the output's own final rounding.
    Returns the max |got - rn(ref)| (0 when every output is the correctly
    rounded oracle value)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mask = ~np.isnan(ref)
    g, r = got[mask], ref[mask]
    d = bar(out_dtype)
    lo, hi = round_to(r - d, out_dtype), round_to(r + d, out_dtype)
    bad = ~((g >= lo) & (g <= hi))
    err = np.abs(g - round_to(r, out_dtype))
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside the bar {d:g}; "
                           f"max |got - rn(ref)| {err.max():.3g}, max |got - ref| "
                           f"{np.abs(g - r).max():.3g}")
    return float(err.max()) if err.size else 0.0
