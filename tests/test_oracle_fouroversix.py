"""Pins of the oracle's FourOverSix block scaling (CPU only).

The pages name a FourOverSix backend and a `model_4o6.pt` NVFP4 checkpoint
(d9249.github.io review, sections on the evidence and on the practical
reading) without defining it.  The rule implemented is a reading: per block,
the usual scale (block maximum -> 6) or the scale that maps the block maximum
to 4, whichever dequantizes with the smaller exact sum of squared errors; equal
errors keep the usual scale.  These tests pin the oracle to that rule written
out independently in exact rational arithmetic (tests/brute.py), to exact ties
constructed by hand, to torch's E4M3 cast for the second candidate's rounding,
and to invariants of the rule."""
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from tests import brute


def _blocks_vs_brute(x, s_g=None):
    """Oracle FourOverSix of x (float32 [rows, k]) against brute force, every block."""
    codes, scales, g = oracle.quantize(x, s_g=s_g, four_over_six=True)
    n4 = 0
    for r in range(x.shape[0]):
        nib = brute.unpack(codes[r])
        for b in range(x.shape[1] // 16):
            blk = [float(v) for v in x[r, 16 * b:16 * b + 16]]
            want_c, want_s, e6, e4 = brute.four_over_six_block(blk, g)
            assert scales[r, b] == want_s, (r, b, scales[r, b], want_s, e6, e4)
            assert nib[16 * b:16 * b + 16] == want_c, (r, b)
            n4 += int(want_s != brute.block_scale(max(abs(v) for v in blk), g))
    return codes, scales, g, n4


def test_block_scale4_matches_torch_e4m3_cast():
    """The second candidate's rounding, RNE_SAT(amax_b / (4 s_g)), against torch's float8_e4m3fn
    cast (a library RNE) of ratios at every E4M3 midpoint and one fp32 ulp either side."""
    vals = np.array([oracle.e4m3_value(b) for b in range(127)])
    mids = (vals[:-1] + vals[1:]) / 2
    ratios = np.concatenate([mids, np.nextafter(mids.astype(np.float32), 0), np.nextafter(mids.astype(np.float32), 1e9),
                             vals, [500.0, 448.0, 1e-9]]).astype(np.float32)
    for s_g in (1.0, 0.25, 2.0 ** -20, 3.0):
        am = (ratios.astype(np.float64) * 4 * s_g).astype(np.float32)
        ok = am.astype(np.float64) == ratios.astype(np.float64) * 4 * s_g  # keep exactly representable products
        ref = torch.from_numpy(np.minimum(ratios[ok], 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = np.array([oracle.block_scale4(a, s_g) for a in am[ok]])
        assert np.array_equal(got, ref), s_g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fouroversix_brute_random(dtype):
    rng = np.random.default_rng(46 if dtype == "f32" else 47)
    x = rng.standard_normal((12, 64)) * np.exp(rng.standard_normal((12, 1)))
    x[rng.random(x.shape) < 0.02] *= 25
    x = x.astype(np.float32)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    _, _, _, n4 = _blocks_vs_brute(x)
    assert n4 >= 5  # the rule picks the second candidate on a fair share of blocks
    for s_g in (np.float32(2.0 ** -6), np.float32(0.0123), np.float32(1e-4)):  # given scales, some saturating
        _blocks_vs_brute(x, s_g)


def test_fouroversix_exact_ties_keep_the_usual_scale():
    """Block [6, b, 0 ...] under s_g = 1: the usual scale is 1.0 (grid 0, .5, 1, 1.5, 2, ...),
    the other 1.5 (grid 0, .75, 1.5, ...); 6 is exact under both.  b = 0.625 lies 1/8 from
    0.5 and from 0.75: an exact tie, which keeps scale 1.0.  Every tie on a fine grid of b
    (up to 8, past the block maximum) keeps the block's usual scale; b just past a tie picks the
    better candidate."""
    ties = 0
    for k in range(0, 8 * 64 + 1):
        b = k / 64.0
        blk = [6.0, b] + [0.0] * 14
        c, sb, e6, e4 = brute.four_over_six_block(blk, 1.0)
        codes, scales, _ = oracle.quantize(np.array([blk], np.float32), s_g=np.float32(1.0), four_over_six=True)
        assert scales[0, 0] == sb and brute.unpack(codes[0]) == c, b
        if e6 == e4:
            ties += 1
            assert sb == brute.block_scale(max(6.0, b), 1.0), b  # the usual scale of this block
    assert ties >= 10
    for b, want in ((0.625, 0x38), (0.63, 0x3C), (0.62, 0x38)):
        _, scales, _ = oracle.quantize(np.array([[6.0, b] + [0.0] * 14], np.float32), s_g=np.float32(1.0),
                                       four_over_six=True)
        assert scales[0, 0] == want, b
    c, sb, e6, e4 = brute.four_over_six_block([6.0, 0.625] + [0.0] * 14, 1.0)
    assert e6 == e4 == F(1, 64)


def test_fouroversix_never_worse_than_the_usual_scale():
    """The kept candidate's exact squared error never exceeds the usual one's, and is strictly
    smaller wherever the second candidate is kept."""
    rng = np.random.default_rng(48)
    x = (rng.standard_normal((16, 48)) * np.exp(2 * rng.standard_normal((16, 3)).repeat(16, axis=1))).astype(np.float32)
    c46, s46, g = oracle.quantize(x, four_over_six=True)
    c6, s6, g6 = oracle.quantize(x)
    assert g == g6
    for r in range(x.shape[0]):
        n46, n6 = brute.unpack(c46[r]), brute.unpack(c6[r])
        for b in range(x.shape[1] // 16):
            blk = [float(v) for v in x[r, 16 * b:16 * b + 16]]
            e46 = brute.sq_err(blk, n46[16 * b:16 * b + 16], s46[r, b], g)
            e6 = brute.sq_err(blk, n6[16 * b:16 * b + 16], s6[r, b], g)
            assert e46 <= e6
            if s46[r, b] != s6[r, b]:
                assert e46 < e6
            else:
                assert n46[16 * b:16 * b + 16] == n6[16 * b:16 * b + 16]


def test_fouroversix_invariants():
    rng = np.random.default_rng(49)
    x = (rng.standard_normal((8, 64)) * 3).astype(np.float32)
    c, s, g = oracle.quantize(x, four_over_six=True)
    # sign symmetry: same scales, every code's sign bit flipped
    cn, sn, gn = oracle.quantize(-x, four_over_six=True)
    assert gn == g and np.array_equal(sn, s) and np.array_equal(cn, c ^ 0x88)
    # power-of-two scaling: s_g scales, the bytes do not change
    for j in (-7, 5):
        cj, sj, gj = oracle.quantize((x * np.float32(2.0 ** j)).astype(np.float32), four_over_six=True)
        assert gj == np.float32(g * 2.0 ** j) and np.array_equal(sj, s) and np.array_equal(cj, c)
    # blocks are independent: permuting blocks permutes the output
    perm = rng.permutation(4)
    xp = x.reshape(8, 4, 16)[:, perm].reshape(8, 64)
    cp, sp, gp = oracle.quantize(xp, s_g=g, four_over_six=True)
    assert np.array_equal(sp, s[:, perm]) and np.array_equal(cp.reshape(8, 4, 8), c.reshape(8, 4, 8)[:, perm])


def test_fouroversix_degenerate_blocks():
    """Zero blocks (and -0) keep scale 0 with sign-only codes; s_g = 0 gives all-zero scales;
    a block on the usual scale's grid keeps it (zero error, and a tie at best)."""
    x = np.zeros((2, 32), np.float32)
    x[0, 3] = -0.0
    x[1, :16] = np.array([6, -4, 3, 2, 1.5, 1, 0.5, 0, 6, 6, -6, 4, 4, 3, 2, 0], np.float32) * np.float32(0.5)
    c, s, g = oracle.quantize(x, s_g=np.float32(0.5 / 448), four_over_six=True)
    c6, s6, _ = oracle.quantize(x, s_g=np.float32(0.5 / 448))
    assert np.array_equal(c, c6) and np.array_equal(s, s6)
    assert s[0].tolist() == [0, 0] and c[0, 1] == 0x80
    z = np.full((1, 16), -1e-3, np.float32)
    cz, sz, gz = oracle.quantize(z, s_g=np.float32(0.0), four_over_six=True)
    assert gz == 0 and sz[0, 0] == 0 and (cz == 0x88).all()


def test_fouroversix_kv_matches_per_head():
    rng = np.random.default_rng(50)
    kv = torch.from_numpy(rng.standard_normal((3, 40, 32)).astype(np.float32) * np.array([1, 10, 0.1])[:, None, None])
    bits = kv.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, hs = oracle.kv_quantize(bits, four_over_six=True)
    for h in range(3):
        c, s, g = oracle.quantize(bits[h], four_over_six=True)
        assert g == hs[h] and np.array_equal(c, codes[h]) and np.array_equal(s, scales[h])
