"""Pins of the oracle's number formats and pool addressing (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from conftest import golden_rows
from oracle import numerics as nx
from oracle import paged


# ---- f16 ---------------------------------------------------------------------------------

def test_f16_rounding_worked_example():
    rows = golden_rows("f16_rounding.txt")
    assert len(rows) == 2
    for row in rows:
        x, want = row[0].split()
        got = int(nx.f32_to_f16(np.float32(float.fromhex(x)))[()])
        assert got == int(want, 16), (x, hex(got), want)


def test_f16_widening_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = nx.f16_to_f32(bits)
    lib = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def test_f16_every_pattern_round_trips():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = nx.f32_to_f16(nx.f16_to_f32(bits))
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    is_nan = (e == 31) & (m != 0)
    assert np.array_equal(back[~is_nan], bits[~is_nan])
    # NaN stays NaN (quiet NaN, same sign)
    bn = back[is_nan]
    assert np.all(((bn >> 10) & 0x1F) == 31) and np.all((bn & 0x3FF) != 0)
    assert np.array_equal(bn >> 15, bits[is_nan] >> 15)


def test_f16_rounding_matches_numpy_on_ties_overflow_subnormals():
    rng = np.random.default_rng(7)
    # exact midpoints between neighbouring f16 values (normal and subnormal), and
    # values a hair above/below them, plus a spread of random magnitudes
    h = np.arange(0, 0x7BFF, dtype=np.uint32).astype(np.uint16)
    lo = nx.f16_to_f32(h).astype(np.float64)
    hi = nx.f16_to_f32(h + 1).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    nudged = np.concatenate([np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    special = np.array([65504.0, 65519.0, 65519.996, 65520.0, 65536.0, 1e6, 2.0 ** -24,
                        2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-10, 0.0, -0.0,
                        np.inf, -np.inf], dtype=np.float32)
    rand = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 12, 200_000))).astype(np.float32)
    for xs in (mids, -mids, nudged, special, rand):
        with np.errstate(over="ignore"):
            lib = xs.astype(np.float16).view(np.uint16)
        ours = nx.f32_to_f16(xs)
        assert np.array_equal(ours, lib)
    assert np.isnan(nx.f16_to_f32(nx.f32_to_f16(np.float32(np.nan))))


def test_f16_relative_error_bound():
    # "Candle model runner" 2.4 "The f16 bound": relative error at most 2^-11 in the normal range
    rng = np.random.default_rng(3)
    x = (rng.uniform(-1, 1, 100_000) * np.exp(rng.uniform(-9, 10, 100_000))).astype(np.float32)
    x = x[(np.abs(x) >= 2.0 ** -14) & (np.abs(x) <= 65504)]
    y = nx.f16_to_f32(nx.f32_to_f16(x)).astype(np.float64)
    rel = np.abs(y - x) / np.abs(x.astype(np.float64))
    assert rel.max() <= 2.0 ** -11


# ---- bf16 --------------------------------------------------------------------------------

@pytest.mark.parametrize("bits,value", [(0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625),
                                        (0x3EAB, 0.333984375), (0x0001, 2.0 ** -133),
                                        (0x7F80, np.inf), (0x8000, -0.0)])
def test_bf16_widening_values(bits, value):
    got = float(nx.bf16_to_f32(np.uint16(bits)))
    assert got == value and np.signbit(got) == np.signbit(value)


# ---- uint4-g32 dequantisation --------------------------------------------------------------

def test_uint4_dequant_is_exact_rational():
    rng = np.random.default_rng(11)
    out, inp = 8, 128
    q = rng.integers(0, 16, size=(out, inp)).astype(np.uint8)
    # bf16 scales spanning many binades, bf16 zero points in [0, 15] with fraction bits
    sc = (rng.uniform(1e-4, 0.05, size=(out, inp // 32))).astype(np.float32)
    zp = rng.uniform(0, 15, size=(out, inp // 32)).astype(np.float32)
    from synthetic import fp32_to_bf16_bits
    sb, zb = fp32_to_bf16_bits(sc), fp32_to_bf16_bits(zp)
    w = nx.dequant_uint4_g32(q, sb, zb)
    scv = nx.bf16_to_f32(sb)
    zpv = nx.bf16_to_f32(zb)
    for o in range(out):
        for i in range(inp):
            g = i // 32
            exact = (Fraction(int(q[o, i])) - Fraction(float(zpv[o, g]))) * Fraction(float(scv[o, g]))
            assert Fraction(float(w[o, i])) == exact


def test_uint4_dequant_group_boundaries():
    # code q, zp and scale of element (o, i) come from group i // 32 of row o
    q = np.full((2, 64), 3, np.uint8)
    from synthetic import fp32_to_bf16_bits
    sb = fp32_to_bf16_bits(np.array([[1.0, 2.0], [4.0, 8.0]], np.float32))
    zb = fp32_to_bf16_bits(np.array([[1.0, 0.0], [2.0, 3.0]], np.float32))
    w = nx.dequant_uint4_g32(q, sb, zb)
    assert np.all(w[0, :32] == 2.0) and np.all(w[0, 32:] == 6.0)
    assert np.all(w[1, :32] == 4.0) and np.all(w[1, 32:] == 0.0)


# ---- symmetric int4-g32 ("Candle model runner" 2.5) ----------------------------------------

def _example_group():
    (row,) = golden_rows("int4_sym_example.txt")
    w = [float(v) for v in row[0].split()]
    return row, np.array([w + [0.0] * (32 - len(w))], np.float32)


def test_int4_sym_chooser_worked_example():
    from synthetic import quantize_int4_sym_g32
    row, w = _example_group()
    q = quantize_int4_sym_g32(w)
    assert int(q.scale[0, 0]) == int(row[2], 16)
    assert float(nx.f16_to_f32(q.scale)[0, 0]) == float(row[1])
    want = [int(v) for v in row[3].split()]
    assert q.q[0, :4].tolist() == want and not q.q[0, 4:].any()
    # the unrounded scale gives another last value: the chooser divides by the stored one
    alt = int(row[4])
    assert int(np.rint(np.float32(w[0, 3]) / np.float32(0.2))) == alt != want[3]


def test_int4_sym_oracle_quantiser_worked_example():
    row, w = _example_group()
    q, sb = nx.quantize_int4_sym_g32(w)
    assert int(sb[0, 0]) == int(row[2], 16)
    assert q[0, :4].tolist() == [int(v) for v in row[3].split()] and not q[0, 4:].any()


def test_int4_sym_oracle_quantiser_bounds_and_generator_agreement():
    # the oracle's quantiser keeps |W - q s| <= s / 2, maps zero groups to zero, and chooses the
    # same values and scales as the input generator's (two writings of section 2.5)
    from synthetic import quantize_int4_sym_g32
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((32, 128)) * rng.uniform(1e-4, 2.0, size=(32, 1))).astype(np.float32)
    w[5, :32] = 0.0
    w[6, 40] = np.float32(2.5) * np.float32(0.25)  # exact multiples of a scale: ties for rint
    q, sb = nx.quantize_int4_sym_g32(w)
    g = quantize_int4_sym_g32(w)
    assert np.array_equal(q, g.q) and np.array_equal(sb, g.scale)
    wh = nx.dequant_int4_sym_g32(q, sb).astype(np.float64)
    s = np.repeat(nx.f16_to_f32(sb).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(w - wh) <= s / 2 * (1 + 1e-6))
    assert not q[5, :32].any() and not sb[5, 0]


def test_int4_sym_dequant_worked_example_is_exact():
    row, w = _example_group()
    s16 = np.array([[int(row[2], 16)]], np.uint16)
    q = np.zeros((1, 32), np.int8)
    q[0, :4] = [int(v) for v in row[3].split()]
    got = nx.dequant_int4_sym_g32(q, s16)
    s = Fraction(row[1])
    assert [Fraction(float(v)) for v in got[0, :4]] == [int(v) * s for v in row[3].split()]
    assert not got[0, 4:].any()
    # 4 * 0.199951171875 etc.: the reconstruction the page's numbers give
    assert got[0, :4].tolist() == [0.7998046875, -1.399658203125, 0.0, 0.39990234375]


def test_int4_sym_dequant_is_exact_rational_and_per_group():
    rng = np.random.default_rng(12)
    out, inp = 6, 96
    q = rng.integers(-8, 8, size=(out, inp)).astype(np.int8)
    sb = rng.uniform(1e-5, 2.0, size=(out, inp // 32)).astype(np.float16).view(np.uint16)
    w = nx.dequant_int4_sym_g32(q, sb)
    sv = sb.view(np.float16)
    for o in range(out):
        for i in range(inp):
            assert Fraction(float(w[o, i])) == int(q[o, i]) * Fraction(float(sv[o, i // 32]))


def test_int4_sym_round_trip_error_bound():
    # |W - q s| <= s / 2 per element (section 2.5), up to the float32 division's rounding
    from synthetic import quantize_int4_sym_g32
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((64, 256)) * rng.uniform(1e-3, 3.0, size=(64, 1))).astype(np.float32)
    w[3, 32:64] = 0.0  # a group of zeros: s = 0, q = 0, exact
    q = quantize_int4_sym_g32(w)
    wh = nx.dequant_int4_sym_g32(q.q, q.scale).astype(np.float64)
    s = np.repeat(nx.f16_to_f32(q.scale).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(w - wh) <= s / 2 * (1 + 1e-6))
    assert not q.q[3, 32:64].any() and not wh[3, 32:64].any()
    assert q.q.min() >= -8 and q.q.max() <= 7
    # symmetric: negating the weights negates the values (rint is odd, no value reaches -8)
    qn = quantize_int4_sym_g32(-w)
    assert np.array_equal(qn.q, -q.q) and np.array_equal(qn.scale, q.scale)


# ---- paged KV pool addressing ----------------------------------------------------------------

def test_kv_address_worked_example():
    (row,) = golden_rows("kv_address.txt")
    B = int(row[0])
    table = [int(v) for v in row[1].split()]
    pos = int(row[2])
    blk, slot = paged.kv_location(pos, table, B)
    assert (blk, slot) == (int(row[3]), int(row[4]))
    D = 128
    for h in range(8):
        assert paged.slab_offset(h, slot, B, D) == (h * 16 + 5) * D
    # in the pool: the block's slab of layer l's K part, then that offset
    n_blocks, Hkv, L = 12, 8, 3
    for layer in range(L):
        for is_v in (False, True):
            off = paged.kv_element_offset(layer, is_v, pos, 3, table, n_blocks, Hkv, B, D)
            slab = B * Hkv * D
            assert off == ((layer * 2 + int(is_v)) * n_blocks + 9) * slab + (3 * 16 + 5) * D
