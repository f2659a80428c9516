"""Oracle codecs: fp16/bf16 rounding, asymmetric INT4, FP8 E4M3 (OCP "fn").

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (8GB page, section 4, "The Hybrid Solution: Sink-FP16 +
Group-Wise Asymmetric INT4 / FP8"):

* FP8 mode casts each 16-bit value to OCP float8_e4m3fn with a per-head
  dynamic scaling factor.
* INT4 mode stores codes q in [0, 15] with an FP16 scale s and an FP16 zero
  point z per head and per group of g elements along the head dimension, and
  reconstructs x = (q - z) * s.
* The kernel pattern of section 7 unpacks two codes per byte: the low nibble
  first (``packed & 0x0F``), then the high nibble (``packed >> 4``).

Readings where the pages are silent:

* INT4 quantize rule, per group of g values held as fp32 (fp16 inputs are
  exact in fp32), every step one IEEE fp32 operation rounded to nearest even:
  ``s = fp16(RN((max - min) / 15))``, replaced by 1 when it rounds to 0;
  ``z = fp16(RN(-min / s))``, clamped to +-65504 when the fp16 rounding
  overflows; ``q = clamp(rint(x / s + z), 0, 15)`` computed against the
  *stored* s and z.  Low nibble = even dimension.
* FP8 scale is per (token, head): ``s = fp16(RN(amax / 448))``, 1 if it
  rounds to 0; code = nearest E4M3 value to ``clamp(x / s, -448, 448)``, ties
  to the even code, sign of zero kept.  Codes 0x7F and 0xFF (NaN) are never
  produced.

The E4M3 values are built from the format definition (1 sign, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 is subnormal with weight 2^-6;
exponent 15 with mantissa 7 is NaN; there is no infinity), and the encoder
searches that value list: a different method from any bit-twiddling encoder.
"""

from __future__ import annotations

import numpy as np

F16_MAX = np.float32(65504.0)
FP8_MAX = 448.0


# ---- plain roundings ---------------------------------------------------------
def to_f16(x):
    """fp32 -> fp16 round-to-nearest-even (numpy's cast is RNE)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def to_bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    bf16 keeps the top 16 bits of fp32; RNE adds 0x7FFF plus the lowest kept
    bit before truncating.  Inputs here are finite.
    """
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f64(bits):
    with np.errstate(invalid="ignore"):  # unwritten pool slots may hold NaN patterns
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- asymmetric INT4 -------------------------------------------------------------
def int4_quantize(x, group):
    """Quantize the last axis of fp16 values ``x`` in groups of ``group``.

    Returns (codes uint8 in [0, 15] with x's shape, scale fp16, zero fp16) with
    scale/zero shaped ``x.shape[:-1] + (D // group,)``.
    """
    x = np.asarray(x, dtype=np.float16)
    d = x.shape[-1]
    if d % group:
        raise ValueError("group must divide the head dimension")
    xg = x.astype(np.float32).reshape(x.shape[:-1] + (d // group, group))
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    s = to_f16(np.float32(mx - mn) / np.float32(15.0))
    s = np.where(s == 0, np.float16(1.0), s)
    s32 = s.astype(np.float32)
    with np.errstate(over="ignore"):
        z32 = (-mn).astype(np.float32) / s32
    z = to_f16(z32)
    z = np.where(np.isinf(z), np.copysign(np.float16(65504.0), z), z).astype(np.float16)
    z32 = z.astype(np.float32)
    with np.errstate(over="ignore"):
        t = xg / s32[..., None]
    t = t + z32[..., None]
    q = np.clip(np.rint(t), 0, 15).astype(np.uint8)
    return q.reshape(x.shape), s, z


def int4_dequant(q, s, z, group):
    """x = (q - z) * s in float64 (exact: every factor has <= 11 significant bits)."""
    q = np.asarray(q).astype(np.float64)
    d = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (d // group, group))
    x = (qg - np.asarray(z, np.float64)[..., None]) * np.asarray(s, np.float64)[..., None]
    return x.reshape(q.shape)


def pack_nibbles(q):
    """Two codes per byte along the last axis: even index low, odd index high."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(p):
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


# ---- FP8 E4M3 (OCP, "fn": finite, no infinities) -------------------------------
def e4m3_value(code):
    """Value of one 8-bit code from the format definition (float64, NaN for NaN)."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes in increasing value order: 0x00 .. 0x7E
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_encode(y):
    """Nearest E4M3 code to each value of ``y`` (|y| <= 448), ties to even code.

    Searches the sorted list of representable magnitudes; at an exact midpoint
    the code with an even mantissa (even code) wins.  Negative values (and -0)
    set the sign bit.
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > FP8_MAX) or np.any(np.isnan(y)):
        raise ValueError("e4m3_encode expects finite |y| <= 448")
    a = np.abs(y)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    neg = np.signbit(y)
    return (code | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def fp8_quantize(x):
    """Quantize the last axis (one (token, head) vector) of fp16 values.

    Returns (codes uint8, scale fp16 with the last axis dropped).
    """
    x = np.asarray(x, dtype=np.float16).astype(np.float32)
    amax = np.abs(x).max(axis=-1)
    s = to_f16(amax / np.float32(FP8_MAX))
    s = np.where(s == 0, np.float16(1.0), s)
    y = x / s.astype(np.float32)[..., None]
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return e4m3_encode(y), s


def fp8_dequant(c, s):
    return E4M3_TABLE[np.asarray(c, dtype=np.uint8)] * np.asarray(s, np.float64)[..., None]
