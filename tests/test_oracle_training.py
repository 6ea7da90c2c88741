"""Pins of the oracle's quantization along rows (quantize_transposed), the
operand layout of the backward GEMMs: exact Fraction brute force over the
columns (tests/brute.py, which never calls the oracle), and the backward
products on inputs that NVFP4 represents exactly, where the reference GEMM
must reduce to numpy's matmul of the inputs themselves."""
import numpy as np
import torch

import oracle
from tests import brute


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(u):
    return (np.asarray(u, np.uint32) << 16).view(np.float32)


def _check_columns_vs_brute(x_f32, x_in=None):
    """quantize_transposed(x) against brute force over the columns of x (blocks of 16 rows)."""
    codes, scales, s_g = oracle.quantize_transposed(x_f32 if x_in is None else x_in)
    cols = [[float(x_f32[r, c]) for r in range(x_f32.shape[0])] for c in range(x_f32.shape[1])]
    bc, bs, bg = brute.quantize(cols)
    assert codes.shape == (x_f32.shape[1], x_f32.shape[0] // 2)
    assert scales.shape == (x_f32.shape[1], x_f32.shape[0] // 16)
    assert float(s_g) == bg
    for c in range(x_f32.shape[1]):
        assert list(scales[c]) == bs[c]
        assert list(codes[c]) == brute.pack(bc[c])


def test_transposed_brute_f32_and_bf16():
    rng = np.random.default_rng(31)
    for rows, cols in [(16, 1), (32, 5), (48, 3)]:
        x = (rng.standard_normal((rows, cols)) * rng.choice([1e-2, 1.0, 30.0])).astype(np.float32)
        x[rng.random(x.shape) < 0.05] *= 20
        _check_columns_vs_brute(x)
        xb = _bf16(x)
        _check_columns_vs_brute(_bf16_to_f32(xb), xb)


def test_transposed_given_scale_saturates_like_row_wise():
    """With a given s_g the blocks are scaled against it; values past 2688 s_g saturate."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((32, 4)).astype(np.float32)
    s_g = np.float32(np.abs(x).max() / 2688 / 4)  # a quarter of the natural scale: the top blocks saturate
    codes, scales, g = oracle.quantize_transposed(x, s_g)
    bc, bs, bg = brute.quantize([[float(x[r, c]) for r in range(32)] for c in range(4)], float(s_g))
    assert g == s_g and [list(s) for s in scales] == bs
    assert [list(c) for c in codes] == [brute.pack(b) for b in bc]
    assert 0x7E in scales  # at least one block saturated at 448


def _on_grid(rng, rows, cols):
    """Values val(code) * 1.75 with a +-10.5 in every 16-row block of every column: the tensor
    amax is 10.5 = 2688 * 2^-8, so s_g = 2^-8, every block scale is 448 exactly and every
    value is representable; quantizing along rows is then lossless."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64) * 1.75
    x = grid[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    for b in range(rows // 16):
        r = 16 * b + rng.integers(0, 16, cols)
        x[r, np.arange(cols)] = 10.5 * rng.choice([-1.0, 1.0], cols)
    return x.astype(np.float32)


def test_backward_products_reduce_to_matmul_on_grid():
    """dX = dY W and dW = dY^T X through the NVFP4 layouts the backward GEMMs use, on exactly
    representable inputs (every block of dY, W, X along the contracted axis holds +-10.5):
    the fp64 reference GEMM must equal numpy's matmul of the inputs.  Square shapes, so an
    operand taken along the wrong axis changes values, not just shapes."""
    rng = np.random.default_rng(33)
    n = 32
    dY = _on_grid(rng, n, n)
    dY[:, :] = np.where(np.arange(n)[None, :] % 16 == 0, 10.5, dY)  # blocks along columns (row-wise) too
    W = _on_grid(rng, n, n)
    X = _on_grid(rng, n, n)
    a = oracle.quantize(dY)
    assert float(a[2]) == 2.0 ** -8
    b = oracle.quantize_transposed(W)
    assert float(b[2]) == 2.0 ** -8 and np.all(b[1] == 0x7E)
    ref, _ = oracle.gemm_ref(*a, *b)
    assert np.array_equal(ref, dY.astype(np.float64) @ W.astype(np.float64))
    ref, _ = oracle.gemm_ref(*oracle.quantize_transposed(dY), *oracle.quantize_transposed(X))
    assert np.array_equal(ref, dY.T.astype(np.float64) @ X.astype(np.float64))
