"""Pins of the oracle codecs (oracle/quant.py).

CPU only.  What pins them, other than themselves:
* the E4M3 value table and encoder against torch.float8_e4m3fn (a library
  implementation of the OCP format), plus the format's saturation rule;
* fp16/bf16 rounding against torch's casts;
* INT4 against a group quantized by hand, closed-form error bounds,
  idempotence, the constant-group special case, and the pages' unpack
  expressions (low nibble = ``p & 0x0F``, high = ``p >> 4``; 8GB page,
  section 7) and byte count (36 bytes per 64 values, 8GB page, section 4).
"""

import numpy as np
import pytest
import torch

from oracle import quant as QT


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = QT.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_including_ties():
    pos = QT.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                  # exact ties
    rnd = np.random.default_rng(0)
    vals = np.concatenate([pos, mids, rnd.uniform(-448, 448, 20000),
                           rnd.uniform(-0.02, 0.02, 20000), -pos, -mids,
                           [0.0, -0.0, 1e-30, -1e-30, 447.99, 448.0]]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = QT.e4m3_encode(vals)
    assert np.array_equal(ref, mine)


def test_e4m3_saturation_and_signed_zero():
    # the format has no infinity; the quantizer clamps to +-448 before encoding
    x = np.array([[1000.0, -1.0, 0.0]], dtype=np.float16)
    c, s = QT.fp8_quantize(x)
    assert s[0] == np.float16(1000.0 / 448.0)
    assert c[0, 0] == 0x7E                          # 1000/s rounds above 448 -> clamp
    assert QT.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert QT.e4m3_encode(np.array([-1e-6]))[0] == 0x80
    assert QT.e4m3_encode(np.array([448.0]))[0] == 0x7E
    with pytest.raises(ValueError):
        QT.e4m3_encode(np.array([449.0]))
    z, s0 = QT.fp8_quantize(np.zeros((1, 8), np.float16))
    assert s0[0] == 1.0 and np.all(z == 0)


def test_fp8_quantize_error_bound():
    rnd = np.random.default_rng(1)
    x = rnd.standard_normal((500, 128)).astype(np.float16)
    c, s = QT.fp8_quantize(x)
    xh = QT.fp8_dequant(c, s)
    amax = np.abs(x.astype(np.float64)).max(axis=1, keepdims=True)
    # relative step of E4M3 is 2^-3 in the normal range -> half-step 2^-4;
    # below 2^-6 * s the absolute step is 2^-9 * s
    err = np.abs(xh - x.astype(np.float64))
    bound = np.maximum(np.abs(x.astype(np.float64)) * 2.0 ** -4, 2.0 ** -10 * s[:, None].astype(np.float64))
    assert np.all(err <= bound * (1 + 1e-3) + 1e-7 * amax)


def test_f16_and_bf16_rounding_match_torch():
    rnd = np.random.default_rng(2)
    x = np.concatenate([rnd.standard_normal(10000) * 10.0 ** rnd.integers(-9, 6, 10000),
                        [65519.0, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, -2.0 ** -25]]).astype(np.float32)
    ref16 = torch.from_numpy(x).to(torch.float16).numpy()
    assert np.array_equal(QT.to_f16(x).view(np.uint16), ref16.view(np.uint16))
    refb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(QT.to_bf16_bits(x), refb)
    assert np.array_equal(QT.bf16_bits_to_f64(refb),
                          torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_int4_hand_worked_group():
    # mn = -1, mx = 2: s = fp16(3/15) = fp16(0.2) = 0.199951171875;
    # z = fp16(1 / s) = fp16(5.00122...) = 5.0;
    # x/s + z = (-0.0012, 5, 7.5006, 15.0024) -> q = (0, 5, 8, 15).
    x = np.array([[-1.0, 0.0, 0.5, 2.0]], dtype=np.float16)
    q, s, z = QT.int4_quantize(x, 4)
    assert s[0, 0] == np.float16(0.199951171875)
    assert z[0, 0] == np.float16(5.0)
    assert q.tolist() == [[0, 5, 8, 15]]
    xh = QT.int4_dequant(q, s, z, 4)
    assert np.allclose(xh, [[-5 * 0.199951171875, 0.0, 3 * 0.199951171875, 10 * 0.199951171875]],
                       rtol=0, atol=0)


@pytest.mark.parametrize("group", [128, 64, 32])
def test_int4_bounds_idempotence_and_range(group):
    rnd = np.random.default_rng(group)
    x = rnd.standard_normal((400, 128)).astype(np.float32)
    x[:, 7] *= 10.0                                    # outlier channel
    x = x.astype(np.float16)
    q, s, z = QT.int4_quantize(x, group)
    assert q.dtype == np.uint8 and q.max() <= 15
    xh = QT.int4_dequant(q, s, z, group)
    sg = np.repeat(s.astype(np.float64), group, axis=-1)
    xd = x.astype(np.float64)
    xg = xd.reshape(400, -1, group)
    straddle = np.repeat((xg.min(-1) <= 0) & (xg.max(-1) >= 0), group, axis=-1)
    # z is -min/s rounded to fp16; groups straddling 0 have |z| <= 15, where
    # fp16 z is within 2^-7 of the exact value: the error stays within s/2 plus that
    err = np.abs(xh - xd)
    assert np.all(err[straddle] <= sg[straddle] * (0.5 + 2.0 ** -7) + 1e-6)
    # re-quantizing the reconstruction with the same (s, z) reproduces q
    qg = np.rint(xh.reshape(400, -1, group).astype(np.float32) / s.astype(np.float32)[..., None]
                 + z.astype(np.float32)[..., None])
    assert np.array_equal(np.clip(qg, 0, 15).astype(np.uint8).reshape(q.shape), q)


def test_int4_constant_group_is_exact():
    x = np.full((3, 64), np.float16(-2.75))
    x[1] = np.float16(0.0)
    x[2] = np.float16(1234.0)
    q, s, z = QT.int4_quantize(x, 64)
    assert np.all(s == 1.0)
    assert np.array_equal(QT.int4_dequant(q, s, z, 64), x.astype(np.float64))


def test_int4_zero_point_stays_finite_for_fp16_inputs():
    # For distinct fp16 values the range is at least one ulp of the minimum,
    # so |min| / s < 15 * 2^11 * 1.5 < 65504: the fp16 zero point never
    # overflows and the +-65504 clamp of the rule is never reached.
    rnd = np.random.default_rng(7)
    base = rnd.choice([-1, 1], 4000) * 2.0 ** rnd.integers(-24, 16, 4000)
    base = base.astype(np.float16)
    ulp = np.abs(np.spacing(base))
    x = np.stack([base, (base.astype(np.float32) + ulp.astype(np.float32)).astype(np.float16)], axis=1)
    x = x[np.isfinite(x).all(axis=1)]
    q, s, z = QT.int4_quantize(x, 2)
    assert np.all(np.isfinite(z)) and np.all(np.abs(z.astype(np.float64)) < 65504)
    assert np.all(np.abs(z.astype(np.float64)) <= 15 * 2 ** 11 * 1.5)


def test_nibble_packing_matches_page_unpack():
    q = np.arange(16, dtype=np.uint8)[::-1].copy()
    p = QT.pack_nibbles(q)
    assert np.array_equal(p & 0x0F, q[0::2])          # low nibble = even index
    assert np.array_equal((p >> 4) & 0x0F, q[1::2])   # high nibble = odd index
    assert np.array_equal(QT.unpack_nibbles(p), q)


def test_int4_bytes_per_group_matches_page():
    # 64 values: 32 bytes of nibbles + fp16 scale + fp16 zero = 36 bytes
    q = np.zeros((1, 64), np.uint8)
    assert QT.pack_nibbles(q).nbytes + 2 + 2 == 36
