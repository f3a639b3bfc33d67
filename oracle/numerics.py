"""Number formats of the decoder -- test infrastructure (oracle).

* bf16 widening: the float32 with bits h << 16
  ("Candle model runner", section 2.3 "The model directory", widening equation).
* f16 widening: (-1)^s 2^(e-15) (1 + m/1024) for 0 < e < 31 and
  (-1)^s 2^-14 m/1024 for e = 0 (same equation); e = 31 is infinity or NaN.
* f32 -> f16: round to nearest, ties to even -- keep the top 10 mantissa bits
  and add one when the dropped bits are above half, or exactly half with the
  kept value odd (same section, last paragraph; worked example in section 3
  "f16 rounding"). Overflow goes to infinity, NaN stays NaN, results below the
  normal range become f16 subnormals.
* uint4-g32 dequantisation W = (q - zp) * scale ("Byte-identical: 1,000 tokens
  of proof", section "The bar we set"), with q a 4-bit code, scale and zp the
  bf16 values of the element's group of 32 input columns. Evaluated in float32
  as t = f32(q) - f32(zp), then w = t * f32(scale), each step rounded to
  nearest even and no fused multiply-add. (With 4-bit q and bf16 zp and scale
  both steps are exact in float32; the tests check that against rational
  arithmetic.)
* symmetric int4-g32 dequantisation W = q * s ("Candle model runner", section
  2.5 "Int4 weights"), q a signed 4-bit value in [-8, 7] and s the f16 scale
  of the element's group of 32 input columns. The product has at most 15
  significant bits, so it is exact in float32 (and in float64). The same
  section's quantisation (the runner's quantise-at-load route) is written out
  too, in float32, with the f32 -> f16 rounding above.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns: the float32 whose bits are h << 16."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32)


def f16_to_f32(bits) -> np.ndarray:
    """Widen f16 bit patterns by the sign/exponent/mantissa formula."""
    h = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (h >> 15) & 1
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + m / 1024.0, (e - 15).astype(np.int64))
    sub = sign * np.ldexp(m / 1024.0, -14)
    out = np.where(e == 0, sub, normal).astype(np.float32)
    # e = 31: infinity (m = 0) or NaN; NaN keeps its sign and mantissa bits
    special = ((s << 31) | 0x7F800000 | (m << 13)).astype(np.uint32).view(np.float32)
    return np.where(e == 31, special, out)


def f32_to_f16(x) -> np.ndarray:
    """Round float32 values to f16 bit patterns, nearest with ties to even."""
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    bits = np.ascontiguousarray(x).reshape(-1).view(np.uint32).astype(np.int64)
    sign = (bits >> 16) & 0x8000
    exp = (bits >> 23) & 0xFF
    man = bits & 0x7FFFFF
    out = np.zeros(bits.shape, dtype=np.int64)

    # NaN keeps a quiet NaN with the top mantissa bits; infinity stays infinity.
    is_special = exp == 0xFF
    nan_payload = np.where(man != 0, 0x200 | (man >> 13), 0)
    out = np.where(is_special, sign | 0x7C00 | nan_payload, out)

    E = exp - 127 + 15  # f16 biased exponent of the value, before rounding

    # Normal f16 range: keep 10 mantissa bits, round on the 13 dropped bits.
    kept = (E << 10) | (man >> 13)
    dropped = man & 0x1FFF
    up = (dropped > 0x1000) | ((dropped == 0x1000) & ((kept & 1) == 1))
    rounded = kept + up.astype(np.int64)  # a carry moves into the exponent by itself
    normal = np.where(rounded >= 0x7C00, 0x7C00, rounded)  # overflow -> infinity
    is_normal = (~is_special) & (E >= 1)
    out = np.where(is_normal, sign | normal, out)

    # Below the normal range: the value is m24 * 2^(E-15-23) with the implicit
    # bit; in units of the f16 subnormal step 2^-24 that is m24 >> (14 - E).
    m24 = np.where(exp == 0, man, man | 0x800000)
    shift = np.clip(14 - E, 14, 40)
    kept_s = np.where(shift >= 25, 0, m24 >> np.minimum(shift, 24))
    mask = (np.int64(1) << shift) - 1
    dropped_s = m24 & mask
    half = np.int64(1) << (shift - 1)
    up_s = (dropped_s > half) | ((dropped_s == half) & ((kept_s & 1) == 1))
    sub = kept_s + up_s.astype(np.int64)
    is_sub = (~is_special) & (E < 1)
    out = np.where(is_sub, sign | sub, out)
    return out.astype(np.uint16).reshape(shape)


def dequant_uint4_g32(q, scale_bits, zp_bits) -> np.ndarray:
    """W = (q - zp) * scale per element, in float32, no fused multiply-add.

    q: uint8 [out, in] codes 0..15 (unpacked); scale_bits, zp_bits: uint16
    [out, in/32] bf16 patterns of each group of 32 input columns.
    """
    q = np.asarray(q)
    out, inp = q.shape
    g = inp // 32
    qf = q.reshape(out, g, 32).astype(np.float32)
    zp = bf16_to_f32(zp_bits).reshape(out, g, 1)
    sc = bf16_to_f32(scale_bits).reshape(out, g, 1)
    t = (qf - zp).astype(np.float32)
    w = (t * sc).astype(np.float32)
    return w.reshape(out, inp)


def quantize_int4_sym_g32(w) -> tuple:
    """Signed int4 values and f16 scale bits per 32-column group ("Candle model runner" 2.5).

    In float32, per group: s = f16(max |W| / 7) (the float32 quotient rounded to nearest even
    in f16), then q = clamp(rint(W / s), -8, 7) with the float32 quotient, rint half to even,
    and s the stored f16 value; a group whose largest magnitude is 0 stores s = 0 and q = 0.
    Returns (q int8 [out, in], scale_bits uint16 [out, in/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    out, inp = w.shape
    grp = w.reshape(out, inp // 32, 32)
    amax = np.max(np.abs(grp), axis=-1)
    s_bits = f32_to_f16((amax / np.float32(7.0)).astype(np.float32))
    s = f16_to_f32(s_bits)[..., None]
    q = np.zeros(grp.shape, dtype=np.int8)
    nz = np.broadcast_to(s > 0, grp.shape)
    ratio = np.divide(grp, s, out=np.zeros_like(grp), where=nz).astype(np.float32)
    q[nz] = np.clip(np.rint(ratio[nz]), -8, 7).astype(np.int8)
    return q.reshape(out, inp), s_bits.reshape(out, inp // 32)


def dequant_int4_sym_g32(q, scale_bits) -> np.ndarray:
    """W = q * s per element, in float32.

    q: int8 [out, in] values -8..7 (unpacked); scale_bits: uint16 [out, in/32] f16 patterns
    of each group of 32 input columns.
    """
    q = np.asarray(q)
    out, inp = q.shape
    g = inp // 32
    sc = f16_to_f32(scale_bits).reshape(out, g, 1)
    w = (q.reshape(out, g, 32).astype(np.float32) * sc).astype(np.float32)
    return w.reshape(out, inp)
