"""The oracle reproduces a hand-worked NVFP4 example (tests/golden/worked_example.json)."""
import json
import math
import os

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def test_worked_example_quantize_dequantize():
    x = np.array([GOLD["x"]], np.float32)
    codes, scales, s_g = oracle.quantize(x)
    assert float(s_g) == GOLD["s_g"]
    assert list(scales[0]) == GOLD["scales"]
    assert list(codes[0]) == GOLD["codes"]
    y = oracle.dequantize(codes, scales, s_g, "f32")[0]
    for got, want in zip(y, GOLD["dequantized"]):
        assert got == want and math.copysign(1, got) == math.copysign(1, want)
    yb = oracle.dequantize(codes, scales, s_g, "bf16")[0]
    assert np.array_equal((yb.astype(np.uint32) << 16).view(np.float32), y)


def test_worked_example_gemm():
    codes = np.array([GOLD["codes"][:8]], np.uint8)
    scales = np.array([[GOLD["scales"][0]]], np.uint8)
    b = np.full((1, 8), 0x22, np.uint8)
    ref, tot = oracle.gemm_ref(codes, scales, GOLD["s_g"], b, np.array([[0x38]], np.uint8), 1.0)
    assert ref[0, 0] == GOLD["gemm_c"]
    assert tot[0, 0] == GOLD["gemm_abssum"]
