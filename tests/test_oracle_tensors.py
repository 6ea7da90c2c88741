"""Pins of the oracle's tensor functions (CPU only): quantize, dequantize,
GEMM reference and KV cache, against exact Fraction brute force
(tests/brute.py), mathematical invariants of the format, and special cases
that reduce to a library routine (numpy matmul)."""
import random
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from tests import brute

E2M1_MIDS = [F(1, 4), F(3, 4), F(5, 4), F(7, 4), F(5, 2), F(7, 2), F(5)]


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(u):
    return (np.asarray(u, np.uint32) << 16).view(np.float32)


def _check_vs_brute(x):
    """x float32 [rows, k]; compare oracle quantize with brute force."""
    codes, scales, s_g = oracle.quantize(x)
    bc, bs, bg = brute.quantize([[float(v) for v in r] for r in x])
    assert float(s_g) == bg
    for r in range(x.shape[0]):
        assert list(scales[r]) == bs[r]
        assert list(codes[r]) == brute.pack(bc[r])
    return codes, scales, s_g


def _adversarial_rows(rng):
    """Rows of fp32 values placed on E2M1 ties, E4M3 ties, underflow, zeros and -0."""
    s_g = F(1, 1024)
    rows = []
    # row 0: the tensor amax (2688 s_g) plus E2M1 ties at scale 448
    S = 448 * s_g
    r0 = [float(6 * S)] + [float(m * S * sg) for m in E2M1_MIDS for sg in (1, -1)] + [-0.0]
    r0 += [float(rng.choice(brute.E2M1_GRID) * S) for _ in range(32 - len(r0))]
    rows.append(r0)
    # row 1: an E4M3 tie (midpoint of 2.0 and 2.25) and an underflowing block
    tie = (F(2) + F(9, 4)) / 2 * 6 * s_g
    r1 = [float(tie)] + [float(tie * F(rng.randrange(-8, 9), 8)) for _ in range(15)]
    under = F(1, 1024) * 6 * s_g  # r == 2^-10 exactly: ties to byte 0
    r1 += [float(under), float(-under / 3)] + [0.0] * 13 + [-0.0]
    rows.append(r1)
    # row 2: E4M3 subnormal scales, just above/below 2^-10 * 6 s_g
    eps = F(1, 2 ** 20)
    r2 = [float(under * (1 + eps))] + [0.0] * 15 + [float(F(3, 1024) * 6 * s_g)] + [float(-F(1, 1024) * 6 * s_g)] * 15
    rows.append(r2)
    return np.array(rows, np.float32)


def test_quantize_brute_random_f32():
    rng = np.random.default_rng(10)
    for shape in [(1, 16), (3, 32), (2, 64), (5, 48)]:
        x = (rng.standard_normal(shape) * rng.choice([1e-3, 1.0, 50.0])).astype(np.float32)
        _check_vs_brute(x)


def test_quantize_brute_bf16_inputs():
    rng = np.random.default_rng(11)
    for shape in [(2, 32), (4, 64)]:
        x = rng.standard_normal(shape).astype(np.float32)
        x[rng.random(shape) < 0.05] *= 20
        xb = _bf16(x)
        codes, scales, s_g = oracle.quantize(xb)
        c2, s2, g2 = _check_vs_brute(_bf16_to_f32(xb))
        assert s_g == g2 and np.array_equal(codes, c2) and np.array_equal(scales, s2)


def test_quantize_brute_adversarial():
    rng = random.Random(12)
    x = _adversarial_rows(rng)
    codes, scales, s_g = _check_vs_brute(x)
    assert s_g == np.float32(2.0 ** -10)
    assert scales[1, 0] == 0x40  # E4M3 tie goes to the even byte
    assert scales[1, 1] == 0x00  # underflowing block
    assert scales[2, 0] == 0x01  # just above 2^-10: smallest subnormal


def test_quantize_all_zero_and_negative_zero():
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = -0.0
    codes, scales, s_g = oracle.quantize(x)
    assert s_g == 0 and not scales.any()
    assert codes[1, 1] == 0x80 and codes.sum() == 0x80


def test_quantize_rejects_bad_shapes_and_nonfinite():
    with pytest.raises(oracle.OracleError):
        oracle.quantize(np.zeros((2, 24), np.float32))
    x = np.zeros((1, 16), np.float32)
    x[0, 5] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quantize(x)


def test_dequantize_brute():
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 256, (3, 32), dtype=np.uint8)
    scales = rng.integers(0, 127, (3, 4), dtype=np.uint8)
    for s_g in (np.float32(1.0), np.float32(0.00123), np.float32(3.3e-7)):
        yb = oracle.dequantize(codes, scales, s_g, "bf16")
        yf = oracle.dequantize(codes, scales, s_g, "f32")
        for r in range(3):
            nib = brute.unpack(codes[r])
            for i in range(64):
                v = brute.dequant_exact(nib[i], scales[r, i // 16], s_g)
                assert yb[r, i] == brute.dequant_bf16_bits(nib[i], scales[r, i // 16], s_g)
                want = brute.round_f32(abs(v))
                assert abs(float(yf[r, i])) == want
                assert (float(yf[r, i]) < 0 or str(float(yf[r, i])) == "-0.0") == bool(nib[i] & 8)


def test_dequantize_single_rounding_differs_from_double():
    # val = 1.5 (code 3), scale byte 0x38 (1.0), s_g chosen so that the exact
    # product lies just above a bf16 midpoint but rounds onto it in fp32.
    s_g = np.float32(F(2 ** 23 + 2 ** 15 + 1, 2 ** 23) / F(3, 2))
    v = F(3, 2) * F(float(s_g))
    assert oracle.dequantize(np.array([[3] + [0] * 7], np.uint8), np.array([[0x38]], np.uint8), s_g, "bf16")[0, 0] \
        == brute.round_bf16_bits(v)


def test_sign_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((16, 128)) * np.exp(rng.standard_normal((1, 128)))).astype(np.float32)
    c, s, g = oracle.quantize(x)
    cn, sn, gn = oracle.quantize(-x)
    assert gn == g and np.array_equal(sn, s) and np.array_equal(cn, c ^ 0x88)
    for j in (-7, 3, 20):
        cj, sj, gj = oracle.quantize((x * np.float32(2.0 ** j)).astype(np.float32))
        assert gj == np.float32(g * 2.0 ** j) and np.array_equal(sj, s) and np.array_equal(cj, c)


def test_block_max_gets_code_seven():
    rng = np.random.default_rng(15)
    x = (rng.standard_normal((32, 256)) * np.exp(2 * rng.standard_normal((32, 1)))).astype(np.float32)
    c, s, g = oracle.quantize(x)
    nib = np.stack([c & 15, c >> 4], -1).reshape(32, 256)
    blocks = np.abs(x).reshape(32, 16, 16)
    arg = blocks.argmax(-1)
    mags = np.take_along_axis((nib & 7).reshape(32, 16, 16), arg[..., None], -1)[..., 0]
    normal = s >= 8
    assert normal.sum() > 100
    assert (mags[normal] == 7).all()


def test_block_and_row_permutation_equivariance():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((8, 96)).astype(np.float32)
    c, s, g = oracle.quantize(x)
    pr = rng.permutation(8)
    pb = rng.permutation(6)
    xp = x[pr].reshape(8, 6, 16)[:, pb].reshape(8, 96)
    cp, sp, gp = oracle.quantize(xp)
    assert gp == g
    assert np.array_equal(sp, s[pr][:, pb])
    assert np.array_equal(cp, c[pr].reshape(8, 6, 8)[:, pb].reshape(8, 48))


def _on_grid(rng, rows, k, e=-5):
    """codes/scales with s_g = 2^e, each block holding a +-6 code, one block at scale 448."""
    codes = rng.integers(0, 16, (rows, k), dtype=np.uint8)
    scales = rng.integers(8, 127, (rows, k // 16), dtype=np.uint8)
    scales[0, 0] = 0x7E
    for r in range(rows):
        for b in range(k // 16):
            codes[r, b * 16 + rng.integers(0, 16)] = rng.choice([7, 15])
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, np.float32(2.0 ** e)


def test_on_grid_round_trip():
    rng = np.random.default_rng(17)
    packed, scales, s_g = _on_grid(rng, 6, 64)
    xf = oracle.dequantize(packed, scales, s_g, "f32")  # exact: <= 6 significant bits
    c, s, g = oracle.quantize(xf)
    assert g == s_g and np.array_equal(s, scales) and np.array_equal(c, packed)
    xb = oracle.dequantize(packed, scales, s_g, "bf16")
    assert np.array_equal(xb, _bf16(xf))  # exact in bf16 too
    c2, s2, g2 = oracle.quantize(xb)
    assert g2 == s_g and np.array_equal(s2, scales) and np.array_equal(c2, packed)


def test_idempotence_on_normal_scale_blocks():
    rng = np.random.default_rng(18)
    x = (rng.standard_normal((16, 128)) * np.exp(1.5 * rng.standard_normal((16, 8)).repeat(16, 1))).astype(np.float32)
    c, s, g = oracle.quantize(x)
    g2 = np.float32(2.0 ** -9)  # replace s_g by a power of two: dequant is then exact in fp32
    y = oracle.dequantize(c, s, g2, "f32")
    c2, s2, gg = oracle.quantize(y)
    assert gg == g2
    normal = s >= 8
    assert np.array_equal(s2[normal], s[normal])
    cb = np.stack([c & 15, c >> 4], -1).reshape(16, 8, 16)
    cb2 = np.stack([c2 & 15, c2 >> 4], -1).reshape(16, 8, 16)
    assert np.array_equal(cb2[normal], cb[normal])


def test_gemm_ref_exact_fraction_dot():
    rng = np.random.default_rng(19)
    M, N, K = 5, 7, 48
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(0, 127, (M, K // 16), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    bsc = rng.integers(0, 127, (N, K // 16), dtype=np.uint8)
    ga, gb = np.float32(0.0371), np.float32(1.7e-3)
    ref, tot = oracle.gemm_ref(ac, asc, ga, bc, bsc, gb)
    for m in range(M):
        an = brute.unpack(ac[m])
        for n in range(N):
            bn = brute.unpack(bc[n])
            terms = [brute.dequant_exact(an[k], asc[m, k // 16], ga) * brute.dequant_exact(bn[k], bsc[n, k // 16], gb)
                     for k in range(K)]
            exact = sum(terms, F(0))
            t = sum((abs(v) for v in terms), F(0))
            assert abs(F(ref[m, n]) - exact) <= F(1, 2 ** 50) * t
            assert abs(F(tot[m, n]) - t) <= F(1, 2 ** 50) * t
    # row / column selection returns the same entries
    r2, t2 = oracle.gemm_ref(ac, asc, ga, bc, bsc, gb, rows=[4, 0], cols=[6, 1, 1])
    assert np.array_equal(r2, ref[[4, 0]][:, [6, 1, 1]])


def test_gemm_ref_reduces_to_matmul_with_unit_scales():
    rng = np.random.default_rng(20)
    M, N, K = 64, 40, 256
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ones_a = np.full((M, K // 16), 0x38, np.uint8)  # E4M3 1.0
    ones_b = np.full((N, K // 16), 0x38, np.uint8)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    A = grid[np.stack([ac & 15, ac >> 4], -1).reshape(M, K)]
    B = grid[np.stack([bc & 15, bc >> 4], -1).reshape(N, K)]
    ref, tot = oracle.gemm_ref(ac, ones_a, 1.0, bc, ones_b, 1.0)
    assert np.array_equal(ref, A @ B.T)
    assert np.array_equal(tot, np.abs(A) @ np.abs(B).T)


def test_gemm_ref_one_hot_b_selects_columns():
    rng = np.random.default_rng(21)
    M, N, K = 9, 4, 64
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(0, 127, (M, K // 16), dtype=np.uint8)
    ga = np.float32(0.25)
    bc = np.zeros((N, K // 2), np.uint8)
    bsc = np.full((N, K // 16), 0x38, np.uint8)
    ks = [0, 17, 38, 63]
    for n, k in enumerate(ks):
        bc[n, k // 2] = 2 << (4 * (k % 2))  # code 2 = 1.0
    ref, _ = oracle.gemm_ref(ac, asc, ga, bc, bsc, 1.0)
    deq = oracle.dequantize(ac, asc, ga, "f32")  # exact: s_g power of two
    for n, k in enumerate(ks):
        assert np.array_equal(ref[:, n], deq[:, k].astype(np.float64))


def test_kv_quantize_per_head_brute_and_structure():
    rng = np.random.default_rng(22)
    H, T, D = 3, 5, 32
    x = rng.standard_normal((H, T, D)).astype(np.float32)
    x[:, :2] *= 8
    x[1] *= 100
    xb = _bf16(x)
    c, s, hs = oracle.kv_quantize(xb)
    xf = _bf16_to_f32(xb)
    for h in range(H):
        bc, bs, bg = brute.quantize([[float(v) for v in r] for r in xf[h]])
        assert float(hs[h]) == bg
        for t in range(T):
            assert list(s[h, t]) == bs[t]
            assert list(c[h, t]) == brute.pack(bc[t])
    perm = [2, 0, 1]
    c2, s2, hs2 = oracle.kv_quantize(xb[perm])
    assert np.array_equal(c2, c[perm]) and np.array_equal(s2, s[perm]) and np.array_equal(hs2, hs[perm])
    out = oracle.kv_dequantize(c, s, hs)
    for h in range(H):
        assert np.array_equal(out[h], oracle.dequantize(c[h], s[h], hs[h], "bf16"))
        nib = brute.unpack(c[h, 2])
        for i in range(D):
            assert out[h, 2, i] == brute.dequant_bf16_bits(nib[i], s[h, 2, i // 16], hs[h])


@pytest.mark.parametrize("case", range(30))
def test_quantize_brute_sweep(case):
    """Seeded random tensors against Fraction brute force: magnitudes from 1e-20 to 1e20,
    values on the quantization grid (every code and most scales a tie), heavy tails with
    zeros, and given scales that make blocks saturate or underflow."""
    rng = np.random.default_rng(500 + case)
    rows, k = int(rng.integers(1, 5)), 16 * int(rng.integers(1, 5))
    kind = case % 3
    if kind == 0:
        x = rng.standard_normal((rows, k)) * 10.0 ** float(rng.integers(-20, 21))
    elif kind == 1:
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 6.0])
        sv = np.array([brute.E4M3_VALUES[b] for b in range(1, 127)], dtype=object)
        s_g = 2.0 ** float(rng.integers(-12, 4))
        blocks = [float(sv[rng.integers(0, 126)]) for _ in range(rows * (k // 16))]
        x = mids[rng.integers(0, len(mids), (rows, k))] * rng.choice([-1.0, 1.0], (rows, k))
        x = x * np.repeat(np.array(blocks).reshape(rows, k // 16), 16, axis=1) * s_g
    else:
        x = rng.standard_normal((rows, k))
        x[rng.random((rows, k)) < 0.05] *= 1000.0
        x[rng.random((rows, k)) < 0.2] = 0.0
    x = x.astype(np.float32)
    if case % 4 == 3:  # a given scale at a random multiple of the computed one
        g = np.float32(oracle.global_scale(oracle.amax(x)) * float(rng.choice([0.01, 0.3, 2.0, 50.0])))
        codes, scales, s_g = oracle.quantize(x, s_g=g)
        bc, bs, bg = brute.quantize([[float(v) for v in r] for r in x], s_g=float(g))
        assert float(s_g) == float(g)
        for r in range(rows):
            assert list(scales[r]) == bs[r]
            assert list(codes[r]) == brute.pack(bc[r])
    else:
        _check_vs_brute(x)
