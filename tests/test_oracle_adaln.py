"""Pins of the oracle's adaLN (orc_adaln) and of its fp64 quantize path, the
reference of the fused adaLN quantizer: torch's fp64 layer_norm (a library
routine) for y, LayerNorm's shift invariance, and exact Fraction brute force
(tests/brute.py) for quantizing fp64 values."""
import numpy as np
import torch

import oracle
from tests import brute


def _mods(rng, groups, k):
    return ((rng.standard_normal((groups, k)) * 0.3).astype(np.float32),
            (rng.standard_normal((groups, k)) * 0.3).astype(np.float32))


def test_adaln_matches_torch_layer_norm_fp64():
    rng = np.random.default_rng(51)
    for rows, k, rpg, eps in [(5, 16, 2, 1e-6), (12, 48, 4, 1e-5), (9, 64, 9, 0.0), (7, 32, 1, 1e-2)]:
        x = (rng.standard_normal((rows, k)) * rng.choice([1e-3, 1.0, 40.0]) + rng.standard_normal((rows, 1))
             ).astype(np.float32)
        groups = (rows + rpg - 1) // rpg
        shift, scale = _mods(rng, groups, k)
        y = oracle.adaln(x, shift, scale, rpg, eps)
        g = np.arange(rows) // rpg
        want = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (k,), eps=eps).numpy()
        want = want * (1.0 + scale[g].astype(np.float64)) + shift[g].astype(np.float64)
        assert np.allclose(y, want, rtol=1e-11, atol=1e-11), np.abs(y - want).max()


def test_adaln_bf16_input_and_shift_invariance():
    """bf16 inputs are read exactly; adding a constant to a row leaves y unchanged up to fp64 rounding."""
    rng = np.random.default_rng(52)
    rows, k = 6, 64
    x = rng.standard_normal((rows, k)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    shift, scale = _mods(rng, 2, k)
    y_b = oracle.adaln(xbits, shift, scale, 3, 1e-6)
    y_f = oracle.adaln(xb.float().numpy(), shift, scale, 3, 1e-6)
    assert np.array_equal(y_b, y_f)
    y_s = oracle.adaln(xb.float().numpy() + np.float32(0.25), shift, scale, 3, 1e-6)  # exact in fp32 here
    assert np.allclose(y_s, y_f, rtol=0, atol=1e-12)
    assert not np.allclose(oracle.adaln(xb.float().numpy() * 2, shift, scale, 3, 1e-6), y_f * 2, atol=1e-3)


def test_quantize_fp64_path_equals_fp32_path_on_fp32_values():
    rng = np.random.default_rng(53)
    x = (rng.standard_normal((9, 64)) * 3).astype(np.float32)
    a = oracle.quantize(x)
    b = oracle.quantize(x.astype(np.float64))
    assert a[2] == b[2] and np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_quantize_fp64_brute():
    """fp64 values that are not fp32 values: s_g from the fp64 amax and every decision exact."""
    rng = np.random.default_rng(54)
    for shape, mag in [((3, 32), 1.0), ((2, 48), 1e-3), ((4, 16), 300.0)]:
        x = rng.standard_normal(shape) * mag
        x[0, 0] = np.nextafter(np.float64(np.float32(x[0, 0])), np.inf)  # certainly not an fp32 value
        codes, scales, s_g = oracle.quantize(x)
        bc, bs, bg = brute.quantize([[float(v) for v in r] for r in x])
        assert float(s_g) == bg
        for r in range(shape[0]):
            assert list(scales[r]) == bs[r] and list(codes[r]) == brute.pack(bc[r])
        g = np.float32(np.abs(x).max() / 2688 / 2)  # a given scale, half the natural one: saturation
        codes, scales, _ = oracle.quantize(x, g)
        bc, bs, _ = brute.quantize([[float(v) for v in r] for r in x], float(g))
        for r in range(shape[0]):
            assert list(scales[r]) == bs[r] and list(codes[r]) == brute.pack(bc[r])
