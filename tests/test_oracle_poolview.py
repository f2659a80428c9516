"""CPU pins of the oracle's pool reader for quantized and sink pools
(``oracle.attention.PoolView``: ``body_codes`` and the INT4 / FP8 / sink
branches of ``block_values``), which the GPU tests use to read back what the
kernels stored.

A pool is written here by hand: the oracle quantizes seeded fp16 tokens
(INT4 groups of 128, 64 or 32; FP8), and their codes, scales, zeros and the
fp16 sink blocks are placed at the byte positions the layout index functions
give (the array offsets are the ones ``test_layout_matches_oracle`` checks
against the library's ``pa_pool_layout``).  What pins the reader:

* read back through ``PoolView`` the codes, scales and zeros come back bit for
  bit, and the sink blocks' fp16 values exactly;
* the logical rebuild is within the quantizers' closed-form error of the
  original values -- INT4: |x - x_hat| <= s/2 plus fp32 rounding (8GB page,
  section 4: x = (q - z) * s); FP8: |x - x_hat| <= s * 2^-4 |y| (+ the
  subnormal step) (three mantissa bits, section 4) -- so a reader that mixes
  up scale and zero, nibble order or token order fails;
* the rebuild does not depend on where the blocks sit (3-minute page,
  "Compartilhamento e compromissos": paging changes no result);
* planted mistakes in the reader (scale and zero arrays swapped, the INT4
  nibbles swapped, the sink arena read as body) make these checks fail.
"""

import numpy as np
import pytest

from oracle import attention as AT
from oracle import layout as LY
from oracle import quant as QT

H, BS = 2, 16


def _tokens(seed, n, D):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, H, D)).astype(np.float32)
    x[:, 1, 3] *= 10.0                               # an outlier channel
    return x.astype(np.float16)


def _write_pool(kind, D, group, seed, nbody=7, nsink=3):
    """One sequence of 1 sink block + nbody - 1 body blocks (the last one
    partial) in a pool of nbody body and nsink sink blocks, blocks at seeded
    physical ids.  Returns (pool bytes, desc, table, length, fp16 tokens,
    per-token codes dict)."""
    rng = np.random.default_rng(seed + 1)
    L = BS * (nbody - 1) + 9
    X = _tokens(seed, L, D)
    dt = LY.DT_INT4 if kind == "int4" else LY.DT_FP8
    arrays, total = LY.pool_arrays(dt, H, D, group, nbody, nsink)
    buf = np.zeros(total, dtype=np.uint8)
    body_ids = rng.permutation(nbody)[: nbody - 1]
    sink_id = int(rng.integers(nsink))
    table = [nbody + sink_id] + [int(b) for b in body_ids]
    codes = {}
    for nm, Xw in (("K", X), ("V", X[::-1].copy())):
        if kind == "int4":
            q, s, z = QT.int4_quantize(Xw, group)
            codes[nm], codes[nm + "S"], codes[nm + "Z"] = q, s, z
        else:
            c, s = QT.fp8_quantize(Xw)
            codes[nm], codes[nm + "S"] = c, s
    views = {nm: LY.array_view(buf, arrays, nm, H, np.uint8) for nm, *_ in arrays}
    for j, pid in enumerate(table):
        toks = np.arange(BS * j, min(BS * j + BS, L))
        n = len(toks)
        for h in range(H):
            if j == 0:                                   # sink block: raw fp16
                for nm, src in (("SK", X), ("SV", X[::-1])):
                    slab = views[nm][pid - nbody, h].view(np.float16)
                    idx = LY.raw_k_index(D) if nm == "SK" else LY.raw_v_index(D)
                    slab[idx[:n]] = src[toks, h]
                continue
            for w in ("K", "V"):
                slab = views[w + "C"][pid, h]
                if kind == "int4":
                    byte, sh = LY.int4_k_byte(D) if w == "K" else LY.int4_v_byte(D)
                    np.bitwise_or.at(slab, byte[:n].ravel(),
                                     (codes[w][toks, h] << sh[:n]).astype(np.uint8).ravel())
                    for m in ("S", "Z"):
                        rows = views[w + m][pid, h].view(np.float16).reshape(BS, -1)
                        rows[:n] = codes[w + m][toks, h]
                else:
                    byte = LY.fp8_k_byte(D) if w == "K" else LY.fp8_v_byte(D)
                    slab[byte[:n].ravel()] = codes[w][toks, h].ravel()
                    views[w + "S"][pid, h].view(np.float16)[:n] = codes[w + "S"][toks, h]
    desc = dict(kv_dtype=dt, n_kv_heads=H, head_dim=D, group_size=group or D, num_blocks=nbody,
                num_sink_blocks=nsink)
    return buf, desc, table, L, X, codes


def _check_reader(buf, desc, table, L, X, codes, kind):
    """The pins listed in the module docstring, for one written pool."""
    view = AT.PoolView(buf, desc)
    g = desc["group_size"]
    body = table[1:]
    toks = np.arange(BS, L)
    for h in range(H):
        got = view.body_codes(body, h)
        for nm, want in codes.items():
            gv = got[nm][: len(toks)]
            if nm.endswith(("S", "Z")):
                assert np.array_equal(gv.view(np.uint16), want[toks, h].view(np.uint16)), nm
            else:
                assert np.array_equal(gv, want[toks, h]), nm
        k0, v0 = view.block_values(table[0], h)
        assert np.array_equal(k0, X[:BS, h].astype(np.float64))
        assert np.array_equal(v0, X[::-1][:BS, h].astype(np.float64))
    K, V = view.logical_kv(table, L)
    for got, src, nm in ((K, X, "K"), (V, X[::-1], "V")):
        x = src.astype(np.float64)
        assert np.array_equal(got[:BS], x[:BS])                 # sink: exact fp16
        err = np.abs(got[BS:] - x[BS:])
        s = codes[nm + "S"][BS:].astype(np.float64)
        if kind == "int4":
            bound = np.repeat(s, g, axis=-1) * (0.5 + 1e-3)
        else:
            bound = s[..., None] * (np.abs(x[BS:]) / s[..., None] * 2.0 ** -4 + 2.0 ** -9) * 1.001
        assert np.all(err <= bound), f"{nm}: rebuild outside the quantizer's error bound"


CASES = [("int4", 128, 128), ("int4", 128, 64), ("int4", 128, 32), ("int4", 64, 32),
         ("fp8", 128, 0), ("fp8", 64, 0)]


@pytest.mark.parametrize("kind,D,group", CASES)
def test_reader_round_trip_and_error_bound(kind, D, group):
    buf, desc, table, L, X, codes = _write_pool(kind, D, group, seed=D + group)
    _check_reader(buf, desc, table, L, X, codes, kind)


@pytest.mark.parametrize("kind,D,group", [("int4", 128, 64), ("fp8", 128, 0)])
def test_rebuild_independent_of_block_placement(kind, D, group):
    """The same blocks moved byte for byte to other ids of a larger pool
    rebuild to the same logical K and V."""
    rng = np.random.default_rng(99)
    buf, desc, table, L, X, codes = _write_pool(kind, D, group, seed=5)
    K, V = AT.PoolView(buf, desc).logical_kv(table, L)
    # move every block to a new id in a larger pool, byte for byte
    nb2, ns2 = desc["num_blocks"] + 4, desc["num_sink_blocks"] + 2
    arrays1, _ = LY.pool_arrays(desc["kv_dtype"], H, D, desc["group_size"], desc["num_blocks"],
                                desc["num_sink_blocks"])
    arrays2, total2 = LY.pool_arrays(desc["kv_dtype"], H, D, desc["group_size"], nb2, ns2)
    buf2 = np.zeros(total2, dtype=np.uint8)
    new_body = rng.permutation(nb2)[: len(table) - 1]
    new_sink = int(rng.integers(ns2))
    table2 = [nb2 + new_sink] + [int(x) for x in new_body]
    for nm, *_ in arrays1:
        v1 = LY.array_view(buf, arrays1, nm, H, np.uint8)
        v2 = LY.array_view(buf2, arrays2, nm, H, np.uint8)
        for j, (p1, p2) in enumerate(zip(table, table2)):
            if (nm in ("SK", "SV")) != (j == 0):
                continue
            o1 = p1 - desc["num_blocks"] if j == 0 else p1
            o2 = p2 - nb2 if j == 0 else p2
            v2[o2] = v1[o1]
    desc2 = dict(desc, num_blocks=nb2, num_sink_blocks=ns2)
    K2, V2 = AT.PoolView(buf2, desc2).logical_kv(table2, L)
    assert np.array_equal(K, K2) and np.array_equal(V, V2)


def _planted(monkeypatch, mistake):
    """Plant one reader mistake in the oracle (on the CPU)."""
    if mistake == "scale-zero-swap":
        orig = LY.array_view

        def swapped(pool_bytes, arrays, name, n, dtype):
            name = {"KS": "KZ", "KZ": "KS", "VS": "VZ", "VZ": "VS"}.get(name, name)
            return orig(pool_bytes, arrays, name, n, dtype)
        monkeypatch.setattr(LY, "array_view", swapped)
    elif mistake == "nibble-swap":
        k0, v0 = LY.int4_k_byte, LY.int4_v_byte
        monkeypatch.setattr(LY, "int4_k_byte", lambda D: (k0(D)[0], 4 - k0(D)[1]))
        monkeypatch.setattr(LY, "int4_v_byte", lambda D: (v0(D)[0], 4 - v0(D)[1]))
    elif mistake == "sink-as-body":
        orig_bv = AT.PoolView.block_values

        def bv(self, bid, head):
            d = dict(self.desc)
            if bid >= d["num_blocks"]:
                return orig_bv(self, bid - d["num_blocks"], head)
            return orig_bv(self, bid, head)
        monkeypatch.setattr(AT.PoolView, "block_values", bv)
    elif mistake == "fp8-scale-swap":
        orig = LY.array_view

        def swapped(pool_bytes, arrays, name, n, dtype):
            name = {"KS": "VS", "VS": "KS"}.get(name, name)
            return orig(pool_bytes, arrays, name, n, dtype)
        monkeypatch.setattr(LY, "array_view", swapped)


@pytest.mark.parametrize("kind,mistake", [("int4", "scale-zero-swap"), ("int4", "nibble-swap"),
                                          ("int4", "sink-as-body"), ("fp8", "fp8-scale-swap"),
                                          ("fp8", "sink-as-body")])
def test_planted_reader_mistakes_are_caught(monkeypatch, kind, mistake):
    D, group = 128, (64 if kind == "int4" else 0)
    buf, desc, table, L, X, codes = _write_pool(kind, D, group, seed=7)
    _check_reader(buf, desc, table, L, X, codes, kind)         # the honest reader passes
    _planted(monkeypatch, mistake)
    with pytest.raises((AssertionError, IndexError, KeyError)):
        _check_reader(buf, desc, table, L, X, codes, kind)


def test_int4_nibble_order_from_the_page():
    """8GB page, section 7 (register unpack): the low nibble of a byte is the
    even element, the high nibble the odd one.  A token whose dims 0 and 1
    quantize to 3 and 12 puts byte 0xC3 where the layout puts dim 0."""
    D = 128
    x = np.zeros((1, 1, D), np.float16)
    x[0, 0, :] = -1.0
    x[0, 0, 0], x[0, 0, 1], x[0, 0, 2] = np.float16(-1.0 + 0.4), np.float16(-1.0 + 1.6), 1.0
    q, s, z = QT.int4_quantize(x, D)
    assert (int(q[0, 0, 0]), int(q[0, 0, 1])) == (3, 12)
    byte, sh = LY.int4_k_byte(D)
    assert byte[0, 0] == byte[0, 1] and (sh[0, 0], sh[0, 1]) == (0, 4)
    packed = QT.pack_nibbles(q[0, 0, :2])
    assert int(packed[0]) == 0xC3
