"""Pins of the oracle's rotary embedding (oracle.rope): the identity at
position 0, the pairwise norm (a rotation), the defining relative-position
property (q . k depends only on the position difference), and the complex
form (x_2i + i x_2i+1) e^(i p th_i) for pair 0 (th_0 = 1)."""
import numpy as np

import oracle


def test_rope_position_zero_is_identity_and_rotations_keep_pair_norms():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((3, 7, 32)).astype(np.float32)
    assert np.array_equal(oracle.rope(x, np.zeros(7)), x.astype(np.float64))
    y = oracle.rope(x, rng.integers(0, 70000, 7))
    n0 = x[..., 0::2].astype(np.float64) ** 2 + x[..., 1::2].astype(np.float64) ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=0)


def test_rope_scores_depend_only_on_position_difference():
    rng = np.random.default_rng(62)
    D = 64
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for m, n, shift in [(5, 2, 100), (0, 4000, 65000), (123, 123, 7)]:
        s1 = (oracle.rope(q, [m]) * oracle.rope(k, [n])).sum()
        s2 = (oracle.rope(q, [m + shift]) * oracle.rope(k, [n + shift])).sum()
        assert abs(s1 - s2) <= 1e-9 * (np.abs(q).sum() * np.abs(k).sum())
    # and it does change with the difference
    assert abs((oracle.rope(q, [10]) * oracle.rope(k, [0])).sum() - (q * k).sum()) > 1e-3


def test_rope_pair_zero_is_complex_rotation_by_position():
    rng = np.random.default_rng(63)
    x = rng.standard_normal((2, 5, 16))
    pos = np.array([0, 1, 2, 1000, 65535])
    y = oracle.rope(x, pos, base=500.0)
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos.astype(np.float64))[None]
    assert np.allclose(y[..., 0], z.real, rtol=0, atol=1e-12) and np.allclose(y[..., 1], z.imag, rtol=0, atol=1e-12)
    # pair i rotates by p * base^(-2i/D): pair 4 of D = 16 at base 500 uses th = 500^-0.5
    z4 = (x[..., 8] + 1j * x[..., 9]) * np.exp(1j * pos * 500.0 ** -0.5)[None]
    assert np.allclose(y[..., 8], z4.real, rtol=0, atol=1e-12)
