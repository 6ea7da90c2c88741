"""GPU parity of nvfp4_adaln_quantize (adaLN fused into the quantizer) with
the oracle's fp64 adaLN followed by its exact quantizer.

The kernel computes y in fp32, so its y differs from the exact y by at most
  tau = 4 * (|1 + a| * (rstd * e_mu + |t| * e_r) + (|t (1 + a)| + |b|) * 2^-23),
  t = (x - mu) * rstd, e_mu = (k / 64 + 8) * 2^-24 * mean|x|, e_r = (k / 64 + 16) * 2^-24
(the fp32 row sums: a sequential sum per lane over k / 64 values and a 6-level
tree across the wave; then sqrt, division, the product and the fma, one rounding each).
With the same s_g on both sides, a scale byte or a code may differ from the
oracle's only where the exact block maximum or element lies within tau of the
decision boundary between the two values; everything else must be identical,
and such elements must be rare.  A computed s_g must be the rounding of a
maximum within tau of the exact one (to one fp32 step), and the codes and scale
bytes computed with it must be the exact quantization of y under that s_g, with
the same near-boundary freedom (when s_g equals the oracle's they must equal
the given-scale call's bytes exactly)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import check_quant_near_exact, dev, f32_bits, log, oracle_input

pytestmark = pytest.mark.gpu

def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _tau(x64, shift, scale, rpg, eps):
    rows, k = x64.shape
    g = np.arange(rows) // rpg
    mu = x64.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x64 - mu) ** 2).mean(axis=1, keepdims=True) + eps)
    t = (x64 - mu) * rstd
    a1 = 1.0 + scale[g].astype(np.float64)
    b = shift[g].astype(np.float64)
    e_mu = (k / 64 + 8) * 2.0 ** -24 * np.abs(x64).mean(axis=1, keepdims=True)
    e_r = (k / 64 + 16) * 2.0 ** -24
    return 4 * (np.abs(a1) * (rstd * e_mu + np.abs(t) * e_r) + (np.abs(t * a1) + np.abs(b)) * 2.0 ** -23)


def _run(x_cpu, shift, scale, rpg, eps, label, check_scale=True):
    nv = _nv()
    y = oracle.adaln(oracle_input(x_cpu), shift.numpy(), scale.numpy(), rpg, eps)
    x64 = x_cpu.double().numpy()
    tau = _tau(x64, shift.numpy(), scale.numpy(), rpg, eps)
    _, _, s_o = oracle.quantize(y)
    xd, shd, scd = x_cpu.to(dev()), shift.to(dev()), scale.to(dev())
    given = nv.adaln_quantize(xd, shd, scd, rpg, eps, s_g=torch.tensor([float(s_o)], device=dev()))
    comp = nv.adaln_quantize(xd, shd, scd, rpg, eps)
    torch.cuda.synchronize()
    check_quant_near_exact(given[0], given[1], y, tau, s_o, label)
    g = comp[2].cpu().numpy()[0]
    if check_scale:
        if f32_bits(g) != f32_bits(s_o):
            # s_g rounds the kernel's max|y|, which lies within tau of the exact maximum
            am, tm = float(np.abs(y).max()), float(tau.max())
            ulp = float(np.spacing(np.float32(s_o)))
            assert (am - tm) / 2688 - ulp <= float(g) <= (am + tm) / 2688 + ulp, (label, g, s_o, tm)
            # and the codes / scale bytes of that call are the exact quantization of y under the
            # kernel's own s_g, up to the same near-boundary freedom
            check_quant_near_exact(comp[0], comp[1], y, tau, g, label + " (computed s_g)")
        else:
            for u, v in zip(comp[:2], given[:2]):
                assert torch.equal(u, v)
    return comp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
# group sizes: one row, a few rows, partial last groups, several workgroups per group, groups
# far longer than the tensor
@pytest.mark.parametrize("rows,k,rpg", [(1, 16, 1), (4, 64, 3), (7, 272, 7), (33, 3072, 8), (9, 4096, 2),
                                        (130, 528, 64), (37, 528, 16), (200, 3072, 50), (1000, 1024, 333),
                                        (20, 64, 1000), (517, 4096, 129)])
def test_adaln_quantize_random(dtype, rows, k, rpg):
    log("adaln_quantize", dtype, rows, k, rpg)
    gen = torch.Generator().manual_seed(rows * 131 + k)
    x = torch.randn(rows, k, generator=gen) * torch.exp(torch.randn(1, k, generator=gen)) + \
        torch.randn(rows, 1, generator=gen)
    G = (rows + rpg - 1) // rpg
    shift = torch.randn(G, k, generator=gen) * 0.3
    scale = torch.randn(G, k, generator=gen) * 0.3
    _run(x.to(dtype), shift, scale, rpg, 1e-6, "random %s %dx%d/%d" % (dtype, rows, k, rpg))


def test_adaln_quantize_degenerate_rows():
    """A constant row (y = shift exactly), a row of one outlier, large eps, an empty call."""
    gen = torch.Generator().manual_seed(9)
    k = 256
    x = torch.randn(6, k, generator=gen)
    x[1] = 0.75
    x[2] = 0.0
    x[2, 17] = 1000.0
    shift = torch.randn(2, k, generator=gen) * 0.3
    scale = torch.randn(2, k, generator=gen) * 0.3
    _run(x.to(torch.bfloat16), shift, scale, 3, 1e-6, "degenerate")
    _run(x.to(torch.bfloat16), shift, scale, 3, 10.0, "large eps")
    nv = _nv()
    s = torch.full((1,), 5.0, device=dev())
    nv.adaln_quantize(torch.empty(0, k, dtype=torch.bfloat16, device=dev()), shift.to(dev()), scale.to(dev()), 3,
                      out=(torch.empty(0, k // 2, dtype=torch.uint8, device=dev()),
                           torch.empty(0, k // 16, dtype=torch.uint8, device=dev())), s_g_out=s)
    torch.cuda.synchronize()
    assert s.item() == 0.0


def test_adaln_quantize_full_size():
    """Pre-norm hidden states [16384, 3072] with per-chunk modulation (4 groups of 4096 tokens)."""
    x, shift, scale, rpg = workloads.adaln_inputs()
    log("adaln full size", tuple(x.shape), "groups", shift.shape[0])
    _run(x, shift, scale, rpg, 1e-6, "full size")


def test_adaln_quantize_deterministic():
    nv = _nv()
    x, shift, scale, rpg = workloads.adaln_inputs(M=2048, K=3072, rows_per_group=512)
    xd, shd, scd = x.to(dev()), shift.to(dev()), scale.to(dev())
    a = nv.adaln_quantize(xd, shd, scd, rpg)
    b = nv.adaln_quantize(xd, shd, scd, rpg)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
