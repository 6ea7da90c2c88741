"""GPU parity of FourOverSix block scaling (NVFP4_FOUR_OVER_SIX) with the
oracle, bit-exact: codes, scale bytes and s_g of nvfp4_quantize (row-wise and
along rows) and of kv_quantize_four_over_six, on ragged small tensors,
hand-built exact ties and degenerate blocks, and at full size on the
activation, weight and KV-cache workloads.  The output is ordinary NVFP4, so
the dequantizer and the GEMM read it unchanged (checked against the oracle)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import (assert_quant_equal, c_to_f64, check_gemm_tiles, dev, log, oracle_input)

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _both(x_cpu, label, s_g=None):
    nv = _nv()
    x = x_cpu.to(dev())
    if s_g is None:
        g = nv.quantize(x, four_over_six=True)
        o = oracle.quantize(oracle_input(x_cpu), four_over_six=True)
    else:
        g = nv.quantize(x, s_g=torch.tensor([s_g], dtype=torch.float32, device=dev()), four_over_six=True)
        o = oracle.quantize(oracle_input(x_cpu), s_g=np.float32(s_g), four_over_six=True)
    torch.cuda.synchronize()
    assert_quant_equal(g, o, label)
    std = oracle.quantize(oracle_input(x_cpu), s_g=o[2])
    share = float((o[1] != std[1]).mean()) if o[1].size else 0.0
    log(label, "blocks on the second candidate scale: %.1f%%" % (100 * share))
    return g, o, share


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,k", [(1, 16), (7, 48), (33, 272), (256, 256), (130, 3072)])
def test_fouroversix_random(dtype, rows, k):
    gen = torch.Generator().manual_seed(rows * 7 + k)
    x = torch.randn(rows, k, generator=gen) * torch.exp(torch.randn(rows, 1, generator=gen))
    x[torch.rand(rows, k, generator=gen) < 0.01] *= 30
    _both(x.to(dtype), "4o6 random %s %dx%d" % (dtype, rows, k))
    _both(x.to(dtype), "4o6 given %s %dx%d" % (dtype, rows, k), s_g=float(np.float32(0.3 / 2688)))


def test_fouroversix_ties_and_degenerate_blocks():
    """Blocks [a, b, 0 ...] with b on a fine grid (every exact tie between the candidates keeps the
    usual scale), the same scaled by powers of two and under a non-power-of-two s_g, zero and -0
    blocks, blocks that underflow the usual scale (byte 0) but not the second one, on-grid blocks
    (exact under the usual scale), and a tiny s_g (the exact slow path)."""
    rows = []
    for k in range(0, 8 * 64 + 1, 2):
        for a in (6.0, 4.5):
            r = [0.0] * 32
            r[0], r[1] = a, k / 64.0
            r[16], r[17] = -a * 2.0 ** -3, -k / 64.0 * 2.0 ** -3
            rows.append(r)
    x = torch.tensor(rows, dtype=torch.float32)
    _, _, share = _both(x, "4o6 tie grid, s_g = 1", s_g=1.0)
    assert 0.05 < share < 0.95
    _both(x, "4o6 tie grid, s_g = 1.3", s_g=1.3)
    _both(x, "4o6 tie grid, tiny s_g", s_g=2.0 ** -120)
    z = torch.zeros(6, 32)
    z[0, 3] = -0.0
    z[1, :16] = torch.tensor([6, -4, 3, 2, 1.5, 1, 0.5, 0, 6, 6, -6, 4, 4, 3, 2, 0]) * 0.5  # on the usual grid
    z[2, :16] = 1.25 * 2.0 ** -10 * 6       # amax_b / (6 s_g) just above 2^-10: usual byte 1
    z[3, :16] = 1.0 * 2.0 ** -10 * 6        # exactly 2^-10: usual byte 0, the other 1.5 2^-10 -> byte 1
    z[4, 1] = 2.0 ** -10 * 6
    z[5] = torch.linspace(-3, 3, 32)
    _both(z, "4o6 degenerate", s_g=1.0)
    _both(z.to(torch.bfloat16), "4o6 degenerate bf16")


@pytest.mark.parametrize("cfg,which", [(2, "A"), (2, "W"), (3, "A"), (3, "W"), (4, "A"), (4, "W")])
def test_fouroversix_config_full_size(cfg, which):
    x = workloads.activations(cfg) if which == "A" else workloads.weights(cfg)
    log("4o6 config", cfg, which, tuple(x.shape))
    _both(x, "4o6 cfg%d %s" % (cfg, which))


def test_fouroversix_kv_cache_full_size():
    """The 24-head KV cache (K and V [24, 65536, 128]) with per-head scales, and its dequantization."""
    nv = _nv()
    k, v = workloads.kv_cache()
    for t, name in ((k, "K"), (v, "V")):
        g = nv.kv_quantize(t.to(dev()), four_over_six=True)
        y = nv.kv_dequantize(*g)
        torch.cuda.synchronize()
        o = oracle.kv_quantize(workloads.bf16_bits(t), four_over_six=True)
        for a, b, lbl in zip(g, o, ("codes", "scales", "head scales")):
            assert np.array_equal(a.cpu().numpy().view(np.uint8), np.asarray(b).view(np.uint8)), name + " " + lbl
        std = oracle.kv_quantize(workloads.bf16_bits(t))
        log("4o6 KV", name, "blocks on the second candidate: %.1f%%" % (100 * float((o[1] != std[1]).mean())))
        yo = oracle.kv_dequantize(*o)
        assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), yo), name + " dequantized"


def test_fouroversix_gemm_and_fused_act():
    """GEMM over FourOverSix operands within the GEMM bound (every tile sampled), and the fused
    activation-quantizing linear with FourOverSix equal to quantize + gemm bit for bit."""
    nv = _nv()
    a, w = workloads.activations(2), workloads.weights(2)
    ad, wd = a.to(dev()), w.to(dev())
    wq = nv.quantize(wd, four_over_six=True)
    c, aq = nv.gemm_fused_act(ad, wq, four_over_six=True)
    aq2 = nv.quantize(ad, four_over_six=True)
    c2 = nv.gemm(aq2, wq)
    torch.cuda.synchronize()
    for u, v_ in zip(aq, aq2):
        assert torch.equal(u, v_)
    assert torch.equal(c, c2)
    ao = oracle.quantize(oracle_input(a), four_over_six=True)
    wo = oracle.quantize(oracle_input(w), four_over_six=True)
    assert_quant_equal(aq, ao, "4o6 fused A")
    assert_quant_equal(wq, wo, "4o6 W")
    check_gemm_tiles(c_to_f64(c), ao, wo, True, "4o6 cfg2 gemm")


@pytest.mark.parametrize("rows,cols", [(48, 5), (272, 65), (784, 516)])
def test_fouroversix_transposed(rows, cols):
    nv = _nv()
    gen = torch.Generator().manual_seed(rows + cols)
    x = (torch.randn(rows, cols, generator=gen) * torch.exp(torch.randn(rows, 1, generator=gen))).to(torch.bfloat16)
    g = nv.quantize_transposed(x.to(dev()), four_over_six=True)
    t = nv.quantize(x.t().contiguous().to(dev()), four_over_six=True)
    torch.cuda.synchronize()
    for u, v_ in zip(g, t):
        assert torch.equal(u, v_)
    assert_quant_equal(g, oracle.quantize_transposed(oracle_input(x), four_over_six=True), "4o6 transposed")
