"""Pins of the oracle's scalar format functions (CPU only).

Checked against what the NVFP4 format fixes, not against the oracle itself:
the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the E4M3FN closed form and
torch's float8_e4m3fn decode/cast (a library routine, RNE, valid up to 448);
exact Fraction brute force (tests/brute.py) for every rounding, with exact
midpoints and their fp32 neighbours.
"""
import math
import random
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from tests import brute



E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_is_the_grid():
    for code in range(16):
        v = oracle.e2m1_value(code)
        mag = E2M1_GRID[code & 7]
        assert abs(v) == mag
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0)
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0  # 0x8 is -0.0


def test_e4m3_decode_closed_form_and_torch():
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = oracle.e4m3_value(b)
        if b & 0x7F == 0x7F:
            assert math.isnan(v) and math.isnan(tv[b])
            continue
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        mag = (1 + m / 8) * 2.0 ** (e - 7) if e else (m / 8) * 2.0 ** -6
        assert v == (-mag if s else mag)
        assert v == tv[b]
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


def _f32(x):
    return float(np.float32(x))


def test_global_scale_brute():
    rng = random.Random(1)
    vals = [0.0, 2688.0, 1.0, 6.0, 448.0, _f32(3.4e38), 2.0 ** -149, 2.0 ** -126, 1e-30, 7.0, 20.0 * 4.5]
    vals += [_f32(rng.lognormvariate(0, 3)) for _ in range(300)]
    vals += [brute.f32_from_bits(rng.randrange(1, 0x7F800000)) for _ in range(300)]
    for a in vals:
        got = float(oracle.global_scale(a))
        want = brute.global_scale(a)
        assert got == want, (a, got, want)
    assert oracle.global_scale(2688.0) == 1.0
    assert oracle.global_scale(0.0) == 0.0


def _e4m3_torch(r):
    t = torch.tensor([min(r, 448.0)], dtype=torch.float32).to(torch.float8_e4m3fn)
    return int(t.view(torch.uint8).item())


def test_block_scale_vs_torch_cast():
    """RNE_SAT(amax_b / (6 s_g)) equals torch's fp32->e4m3fn cast of the ratio (clamped to 448)."""
    rng = random.Random(2)
    rs = [rng.uniform(0, 500) for _ in range(400)] + [2.0 ** rng.uniform(-12, 9) for _ in range(400)]
    vals = brute.E4M3_VALUES
    for i in range(126):  # every midpoint and its fp32 neighbours
        mid = float((vals[i] + vals[i + 1]) / 2)
        rs += [mid, float(np.nextafter(np.float32(mid), np.float32(0))), float(np.nextafter(np.float32(mid), np.float32(1e9)))]
    rs += [448.0, 460.0, 464.0, 1e4, 2.0 ** -10, 2.0 ** -11, 1.5 * 2.0 ** -10]
    for r in rs:
        r = _f32(r)
        for s_g in (0.5, _f32(1 / 2688.0), _f32(0.0123), _f32(3.7e-5)):
            amax_b = float(F(r) * 6 * F(s_g))  # exact in fp64 (<= 50 bits)
            assert F(amax_b) == F(r) * 6 * F(s_g)
            assert oracle.block_scale(amax_b, s_g) == _e4m3_torch(r), (r, s_g)


def test_block_scale_brute_fp32_inputs():
    rng = random.Random(3)
    for _ in range(1500):
        s_g = _f32(2.0 ** rng.uniform(-20, 5))
        amax_b = _f32(s_g * 6 * 2.0 ** rng.uniform(-12, 10))
        assert oracle.block_scale(amax_b, s_g) == brute.block_scale(amax_b, s_g)
    assert oracle.block_scale(0.0, 1.0) == 0
    assert oracle.block_scale(1.0, 0.0) == 0


def test_block_scale_exact_ties_go_to_even_byte():
    vals = brute.E4M3_VALUES
    s_g = 0.25
    for i in range(126):
        mid = (vals[i] + vals[i + 1]) / 2
        amax_b = float(mid * 6 * F(s_g))
        want = i if i % 2 == 0 else i + 1
        assert oracle.block_scale(amax_b, s_g) == want


def test_e2m1_code_midpoints_and_neighbours():
    mids = [F(1, 4), F(3, 4), F(5, 4), F(7, 4), F(5, 2), F(7, 2), F(5)]
    tie_to = [0, 2, 2, 4, 4, 6, 6]  # even code of each tie
    for S in (F(1), F(3, 2) * F(2) ** -7, F(15, 8) * F(_f32(0.0371))):
        for m, t in zip(mids, tie_to):
            x = m * S
            xf = float(x)
            assert F(xf) == x
            assert oracle.e2m1_code(xf, float(S)) == t
            assert oracle.e2m1_code(-xf, float(S)) == 8 | t
            for nb in (np.nextafter(xf, 0.0), np.nextafter(xf, 1e9)):
                assert oracle.e2m1_code(float(nb), float(S)) == brute.e2m1_code(float(nb), S)


def test_e2m1_code_brute_random_and_saturation():
    rng = random.Random(4)
    for _ in range(3000):
        S = F(_f32(2.0 ** rng.uniform(-10, 3))) * brute.E4M3_VALUES[rng.randrange(1, 127)]
        x = _f32(rng.uniform(-8, 8) * float(S))
        assert oracle.e2m1_code(x, float(S)) == brute.e2m1_code(x, S), (x, S)
    assert oracle.e2m1_code(1e30, 1.0) == 7
    assert oracle.e2m1_code(-7.0, 1.0) == 15
    assert oracle.e2m1_code(-0.0, 1.0) == 8
    assert oracle.e2m1_code(-0.1, 1.0) == 8  # negative that rounds to zero keeps its sign
    assert oracle.e2m1_code(0.3, 0.0) == 0 and oracle.e2m1_code(-0.3, 0.0) == 8


def test_round_bf16_vs_torch_and_brute():
    rng = random.Random(5)
    xs = [brute.f32_from_bits(rng.randrange(0, 0x7F000000)) for _ in range(2000)]
    xs += [(1.0 + k * 2.0 ** -7 + 2.0 ** -8) * 2.0 ** e for k in range(8) for e in (-130, -20, 0, 9)]  # exact bf16 ties
    t = torch.tensor(xs, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, want in zip(xs, t):
        assert oracle.round_bf16(x) == int(want)
        assert oracle.round_bf16(-x) == int(want) | 0x8000
    # values with more than 24 significant bits: fp32 double rounding would differ
    for _ in range(2000):
        v = F(rng.randrange(1, 2 ** 30)) * F(2) ** rng.randrange(-60, 20)
        assert oracle.round_bf16(float(v)) == brute.round_bf16_bits(v)
    v = F(1) + F(1, 256) + F(1, 2 ** 29)  # just above a bf16 midpoint, rounds to midpoint in fp32
    assert oracle.round_bf16(float(v)) == brute.round_bf16_bits(v) == 0x3F81
    assert oracle.round_bf16(-0.0) == 0x8000
