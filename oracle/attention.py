"""Oracle decode attention: rebuild each sequence's logical K/V through its block
table, then run textbook softmax attention in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The definition followed:

* Paging changes neither the computation nor the model's results; only the
  layout and the fetch of the cache change (3-minute page, "Compartilhamento e
  compromissos" and "A analogia com memoria virtual").  So the result is plain
  attention over the logically contiguous cache.
* Logical block i holds tokens 16i .. 16i+15 and sits at physical block
  ``table[i]`` (8GB page, section 3, "How Logical-to-Physical Block Tables
  Work"); the kernel gathers K for the QK^T dot product and V for the
  softmax-weighted sum through that table (same section).
* Grouped-query attention: 32 query heads share 8 KV heads (8GB page,
  section 2, variable list).  Reading: query head h uses KV head
  ``h // (Hq // Hkv)``.
* One new query per sequence attends to all ``seq_len`` cached tokens (its own
  K/V already appended), with no extra mask.  ``seq_len == 0`` gives a zero
  output row.  The softmax scale is passed in (1/sqrt(head_dim) throughout).
"""

from __future__ import annotations

import numpy as np

from . import layout as LY
from . import quant as QT


def attention_one(q, K, V, scale):
    """Textbook attention for one sequence.

    q: [Hq][D]; K, V: [L][Hkv][D] (any float dtype; computed in float64).
    Returns [Hq][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, d = q.shape
    L, hkv, _ = K.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if L == 0:
        return out
    group = hq // hkv
    for h in range(hq):
        g = h // group
        s = scale * (K[:, g, :] @ q[h])
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ V[:, g, :]
    return out


def verify_attention_one(q, K, V, scale):
    """Attention of a speculative verify step for one sequence.

    The target model scores the gamma + 1 new tokens (the last accepted one
    and the gamma draft tokens) in one pass (8GB page, section 6,
    "Speculative Decoding: Breaking the Bandwidth Wall").  Reading: their K/V
    are already appended, so they are the last ``nq`` of the ``L`` cached
    tokens, and query i sees the cache up to and including its own token,
    tokens ``0 .. L - nq + i`` (causal among the new tokens).  A query whose
    position lies before the cache start sees nothing: zero row.

    q: [nq][Hq][D]; K, V: [L][Hkv][D].  Returns [nq][Hq][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    nq = q.shape[0]
    L = np.asarray(K).shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(nq):
        n = L - nq + i + 1
        if n > 0:
            out[i] = attention_one(q[i], np.asarray(K)[:n], np.asarray(V)[:n], scale)
    return out


def causal_attention(q, K, V, scale):
    """Causal self-attention of a whole prompt in one pass: token i's query
    sees tokens 0..i.  Written as one masked score matrix (the form that
    chunked prefill avoids materializing: 8GB page, section 5, "Notice two
    critical details", item 1 "Chunked Prefill"), independently of the
    per-query loops above.

    q: [P][Hq][D]; K, V: [P][Hkv][D].  Returns [P][Hq][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    P, hq, _ = q.shape
    hkv = K.shape[1]
    group = hq // hkv
    out = np.zeros(q.shape, dtype=np.float64)
    future = np.triu(np.ones((P, P), dtype=bool), k=1)  # key t > query i
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ K[:, g, :].T)          # [P][P]
        s[future] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
    return out


def prefill_chunks(q, K, V, scale, chunk):
    """A prompt prefilled in chunks of `chunk` tokens (8GB page, section 5,
    "Notice two critical details", item 1 "Chunked Prefill"):
    chunk c's K/V join the cache, then its queries attend over the cache so
    far, causally among themselves -- the verify step's operation with
    n_query = the chunk's length.  Returns [P][Hq][D] float64."""
    P = np.asarray(q).shape[0]
    parts = []
    for s0 in range(0, P, chunk):
        e = min(P, s0 + chunk)
        parts.append(verify_attention_one(np.asarray(q)[s0:e], np.asarray(K)[:e], np.asarray(V)[:e], scale))
    return np.concatenate(parts) if parts else np.zeros(np.asarray(q).shape)


def decode_attention(q, kv, scale):
    """q: [B][Hq][D]; kv: list of (K, V) per sequence, each [L_b][Hkv][D]."""
    return np.stack([attention_one(q[b], K, V, scale) for b, (K, V) in enumerate(kv)])


class PoolView:
    """Read a pool's bytes (copied back from the device) through the layout.

    ``desc`` is a dict with the descriptor fields (kv_dtype, n_kv_heads,
    head_dim, group_size, num_blocks, num_sink_blocks, sink_blocks_per_seq).
    """

    def __init__(self, pool_bytes, desc):
        self.b = np.asarray(pool_bytes, dtype=np.uint8)
        self.desc = desc
        self.bs = desc.get("block_size", LY.BLOCK)
        self.arrays, self.total = LY.pool_arrays(
            desc["kv_dtype"], desc["n_kv_heads"], desc["head_dim"],
            desc.get("group_size", desc["head_dim"]), desc["num_blocks"],
            desc.get("num_sink_blocks", 0), self.bs)

    def _view(self, name, dtype):
        return LY.array_view(self.b, self.arrays, name, self.desc["n_kv_heads"], dtype)

    def _raw_dtype(self):
        kd = self.desc["kv_dtype"]
        return {LY.DT_F32: np.float32, LY.DT_F16: np.float16, LY.DT_BF16: np.uint16}[kd]

    def _to64(self, x, kd):
        if kd == LY.DT_BF16:
            return QT.bf16_bits_to_f64(x)
        return np.asarray(x).astype(np.float64)

    def body_codes(self, ids, head):
        """Logical per-token codes and metadata of body blocks ``ids``."""
        D = self.desc["head_dim"]
        kd = self.desc["kv_dtype"]
        if kd == LY.DT_INT4:
            out = {w: LY.gather_int4_codes(self._view(w + "C", np.uint8), ids, head, D, w)
                   for w in ("K", "V")}
            for nm in ("KS", "KZ", "VS", "VZ"):
                out[nm] = LY.gather_rows(self._view(nm, np.float16), ids, head)
            return out
        if kd == LY.DT_FP8:
            out = {w: LY.gather_fp8_codes(self._view(w + "C", np.uint8), ids, head, D, w)
                   for w in ("K", "V")}
            for nm in ("KS", "VS"):
                out[nm] = LY.gather_rows(self._view(nm, np.float16), ids, head)[:, 0]
            return out
        raise ValueError("body_codes is for quantized pools")

    def block_values(self, bid, head):
        """K, V of one physical block and head as float64 [bs][D] each."""
        desc = self.desc
        D, N = desc["head_dim"], desc["num_blocks"]
        kd = desc["kv_dtype"]
        if bid >= N:  # sink arena: raw fp16
            sk = self._view("SK", np.float16)
            sv = self._view("SV", np.float16)
            return (LY.gather_raw(sk, [bid - N], head, D, "K").astype(np.float64),
                    LY.gather_raw(sv, [bid - N], head, D, "V").astype(np.float64))
        if kd in LY.ELEM:
            dt = self._raw_dtype()
            k = LY.gather_raw(self._view("K", dt), [bid], head, D, "K", self.bs)
            v = LY.gather_raw(self._view("V", dt), [bid], head, D, "V", self.bs)
            return self._to64(k, kd), self._to64(v, kd)
        c = self.body_codes([bid], head)
        if kd == LY.DT_INT4:
            g = desc["group_size"]
            return (QT.int4_dequant(c["K"], c["KS"], c["KZ"], g),
                    QT.int4_dequant(c["V"], c["VS"], c["VZ"], g))
        return QT.fp8_dequant(c["K"], c["KS"]), QT.fp8_dequant(c["V"], c["VS"])

    def logical_kv(self, table_row, seq_len):
        """Rebuild [L][Hkv][D] float64 K and V of one sequence."""
        H, D, bs = self.desc["n_kv_heads"], self.desc["head_dim"], self.bs
        nblk = (seq_len + bs - 1) // bs
        K = np.zeros((nblk * bs, H, D))
        V = np.zeros((nblk * bs, H, D))
        for j in range(nblk):
            for h in range(H):
                k, v = self.block_values(int(table_row[j]), h)
                K[j * bs:(j + 1) * bs, h] = k
                V[j * bs:(j + 1) * bs, h] = v
        return K[:seq_len], V[:seq_len]
