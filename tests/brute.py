"""Exact brute-force NVFP4 reference with fractions.Fraction, for pinning the oracle.

Written independently of oracle/: it never calls it and takes every rounding
as "the nearest value of an explicitly enumerated table, ties to the even
entry", with distances computed in exact rational arithmetic.  Only for tiny
inputs.

Tables: the E2M1 magnitudes are the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} in code
order (OCP Microscaling v1.0 E2M1: bit 3 sign, bits 2:0 the magnitude index);
the E4M3FN values are enumerated from its definition (bias 7, 3 mantissa
bits, subnormals 2^-6 * m/8, byte 0x7F is NaN so the finite non-negative
values are bytes 0x00..0x7E).
"""
from fractions import Fraction as F
import math
import struct

E2M1_GRID = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def _e4m3_table():
    vals = []
    for b in range(127):
        e, m = b >> 3, b & 7
        if e == 0:
            vals.append(F(m, 8) * F(1, 64))
        else:
            vals.append((1 + F(m, 8)) * (F(2) ** (e - 7)))
    return vals


E4M3_VALUES = _e4m3_table()


def nearest_even(table, v):
    """Index of the entry of a sorted table nearest to v >= 0; ties to the even index."""
    best, best_d = None, None
    for i, t in enumerate(table):
        d = abs(v - t)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def _f32_neighbours(x):
    """fp32 values around a Python float x (exact float32 conversion may round)."""
    c = struct.unpack("<f", struct.pack("<f", x))[0]
    u = f32_bits(c)
    out = {c}
    for d in (-2, -1, 1, 2):
        v = u + d
        if 0 <= v < 0x7F800000:
            out.add(f32_from_bits(v))
    return sorted(out)


def round_f32(v):
    """Exact RNE of a non-negative Fraction to fp32 (no overflow handling needed here)."""
    assert v >= 0
    if v == 0:
        return 0.0
    cands = _f32_neighbours(float(v))
    best, best_d = None, None
    for c in cands:
        d = abs(F(c) - v)
        if best is None or d < best_d or (d == best_d and (f32_bits(c) & 1) == 0):
            best, best_d = c, d
    return best


def round_bf16_bits(v):
    """Exact RNE of a Fraction to bfloat16, as a bit pattern (finite range only)."""
    neg = v < 0
    a = -v if neg else v
    sign = 0x8000 if neg else 0
    if a == 0:
        return sign
    # exponent of the leading bit
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    ulp = F(2) ** (max(e, -126) - 7)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > F(1, 2) or (rem == F(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    return sign | (f32_bits(float(r)) >> 16)


def global_scale(amax):
    return round_f32(F(float(amax)) / 2688)


def block_scale(amax_b, s_g):
    if s_g == 0 or amax_b == 0:
        return 0
    return nearest_even(E4M3_VALUES, F(float(amax_b)) / (6 * F(float(s_g))))


def e2m1_code(x, S):
    sign = 8 if math.copysign(1.0, float(x)) < 0 else 0
    if S == 0:
        return sign
    return sign | nearest_even(E2M1_GRID, abs(F(float(x))) / F(S))


def quantize(rows, s_g=None):
    """rows: list of lists of Python floats (exact fp32/bf16 values).

    Returns (codes as list of lists of nibbles, scales list of lists, s_g)."""
    if s_g is None:
        amax = max((abs(v) for r in rows for v in r), default=0.0)
        s_g = global_scale(amax)
    codes, scales = [], []
    for r in rows:
        cr, sr = [], []
        for j in range(0, len(r), 16):
            blk = r[j:j + 16]
            sb = block_scale(max(abs(v) for v in blk), s_g)
            S = E4M3_VALUES[sb] * F(float(s_g))
            sr.append(sb)
            cr.extend(e2m1_code(v, S) for v in blk)
        codes.append(cr)
        scales.append(sr)
    return codes, scales, s_g


def e2m1_value(code):
    v = E2M1_GRID[code & 7]
    return -v if code & 8 else v


def dequant_exact(code, sb, s_g):
    return e2m1_value(int(code)) * E4M3_VALUES[int(sb)] * F(float(s_g))


def pack(nibbles):
    return [nibbles[i] | (nibbles[i + 1] << 4) for i in range(0, len(nibbles), 2)]


def unpack(byte_row):
    out = []
    for b in byte_row:
        out.append(int(b) & 15)
        out.append(int(b) >> 4)
    return out


def dequant_bf16_bits(code, sb, s_g):
    """bf16 bits of RN(val(code) val(sb) s_g); the code's sign bit is kept for zeros."""
    v = abs(dequant_exact(code, sb, s_g))
    return round_bf16_bits(v) | (0x8000 if int(code) & 8 else 0)


def block_scale4(amax_b, s_g):
    """E4M3 byte nearest to amax_b / (4 s_g), ties to the even byte (the FourOverSix candidate
    that maps the block maximum to 4)."""
    if s_g == 0 or amax_b == 0:
        return 0
    return nearest_even(E4M3_VALUES, F(float(amax_b)) / (4 * F(float(s_g))))


def sq_err(blk, codes, sb, s_g):
    """Exact sum of squared differences between a block and its dequantized codes."""
    return sum((F(float(v)) - dequant_exact(c, sb, s_g)) ** 2 for v, c in zip(blk, codes))


def four_over_six_block(blk, s_g):
    """FourOverSix reading for one 16-value block under s_g: encode with the scale for 6 and
    with the scale for 4, keep the one with the smaller exact squared error (ties: 6).
    Returns (nibbles, scale byte, err6, err4)."""
    amax_b = max(abs(v) for v in blk)
    out = []
    for sb in (block_scale(amax_b, s_g), block_scale4(amax_b, s_g)):
        S = E4M3_VALUES[sb] * F(float(s_g))
        codes = [e2m1_code(v, S) for v in blk]
        out.append((codes, sb, sq_err(blk, codes, sb, s_g)))
    (c6, s6, e6), (c4, s4, e4) = out
    return (c4, s4, e6, e4) if e4 < e6 else (c6, s6, e6, e4)
