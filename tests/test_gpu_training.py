"""GPU parity of nvfp4_quantize_transposed (NVFP4 of x^T, blocks along the rows
of x) with the oracle, bit-exact, and of the backward GEMMs of a linear that
take those operands (dX = dY W, dW = dY^T X) within the GEMM bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_quant_equal, c_to_f64, check_gemm_bound, check_gemm_tiles, dev, log, \
    oracle_input

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _both(x_cpu, label, s_g=None):
    nv = _nv()
    x = x_cpu.to(dev())
    if s_g is None:
        g = nv.quantize_transposed(x)
        o = oracle.quantize_transposed(oracle_input(x_cpu))
    else:
        g = nv.quantize_transposed(x, s_g=torch.tensor([s_g], dtype=torch.float32, device=dev()))
        o = oracle.quantize_transposed(oracle_input(x_cpu), s_g=np.float32(s_g))
    torch.cuda.synchronize()
    assert_quant_equal(g, o, label)
    return g, o


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(16, 1), (16, 3), (48, 5), (256, 64), (272, 65), (512, 130), (4096, 3),
                                       (784, 516), (48, 8), (272, 264), (528, 2048), (784, 2056), (2048, 1024),
                                       (2032, 1020)])
def test_transposed_random(dtype, rows, cols):
    """Tile edges in both directions, cols % 4 != 0 (scalar loads), one-block columns, and row
    and column tiles both in eights (the XCD tile order: 2048 x 1024, and 2032 x 1020 with
    ragged last tiles) or not."""
    log("quantize_transposed", dtype, rows, cols)
    gen = torch.Generator().manual_seed(rows * 31 + cols)
    x = torch.randn(rows, cols, generator=gen) * torch.exp(torch.randn(rows, 1, generator=gen))
    x[torch.rand(rows, cols, generator=gen) < 0.01] *= 30
    _both(x.to(dtype), "random %s %dx%d" % (dtype, rows, cols))


def test_transposed_given_scale_zeros_and_empty():
    log("quantize_transposed given scale / zeros / empty")
    gen = torch.Generator().manual_seed(41)
    x = torch.randn(64, 40, generator=gen)
    _both(x, "given (saturating)", s_g=float(np.float32(0.4 / 2688)))
    z = torch.zeros(32, 8)
    z[3, 1] = -0.0
    z[20:, 5] = 1e-3
    z[0:16, 6] = -1e-9  # blocks that underflow to scale byte 0
    _both(z, "zeros / -0 / underflow")
    _both(torch.zeros(32, 0), "no columns")


def test_transposed_equals_quantize_of_transpose_on_gpu():
    """Same bytes as the row-wise quantizer on a transposed copy (both on the GPU)."""
    nv = _nv()
    x = workloads.activations(2, M=1040, K=776).to(dev())
    a = nv.quantize_transposed(x)
    b = nv.quantize(x.t().contiguous())
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("which", ["W", "A", "dY"])
def test_transposed_config3_full_size_sampled_columns(which):
    """The FFN up-projection's backward operands at full size, W [14336, 3072],
    A [16384, 3072] and dY [16384, 14336] quantized along their rows: s_g from
    the whole tensor, and sampled columns bit-exact to the oracle."""
    x_cpu = {"W": lambda: workloads.weights(3), "A": lambda: workloads.activations(3),
             "dY": lambda: workloads.output_grads(3)}[which]()
    log("cfg3", which, tuple(x_cpu.shape))
    nv = _nv()
    codes, scales, s_g = nv.quantize_transposed(x_cpu.to(dev()))
    torch.cuda.synchronize()
    xo = oracle_input(x_cpu)
    want_g = np.float32(oracle.global_scale(oracle.amax(xo)))
    assert s_g.cpu().numpy()[0].view(np.uint32) == want_g.view(np.uint32)
    rows, cols = x_cpu.shape
    rng = np.random.default_rng(len(which))
    sel = np.unique(np.concatenate([[0, 1, cols - 1], rng.integers(0, cols, 13)]))
    oc, os_, _ = oracle.quantize_transposed(np.ascontiguousarray(xo[:, sel]), want_g)
    assert_quant_equal((codes[sel], scales[sel], s_g), (oc, os_, want_g), "cfg3 %s columns" % which)


def _small_backward(seed, M, N, K):
    a = workloads.activations(3, M=M, K=K)
    w = workloads.weights(3, N=N, K=K)
    dy = workloads.output_grads(3, M=M, N=N)
    return a, w, dy


@pytest.mark.parametrize("M,N,K", [(48, 32, 16), (272, 160, 96), (1024, 768, 512)])
def test_backward_gemms_small(M, N, K):
    """dX = dY W (A = dY row-wise, B = W along rows) and dW = dY^T A (both along rows), every
    output against the oracle's fp64 reference."""
    nv = _nv()
    a, w, dy = _small_backward(M + N + K, M, N, K)
    log("backward", M, N, K)
    ad, wd, dyd = a.to(dev()), w.to(dev()), dy.to(dev())
    dyq, wtq = nv.quantize(dyd), nv.quantize_transposed(wd)
    dx = nv.gemm(dyq, wtq, out_dtype=torch.float32)  # [M, K]
    dytq, atq = nv.quantize_transposed(dyd), nv.quantize_transposed(ad)
    dw = nv.gemm(dytq, atq, out_dtype=torch.bfloat16)  # [N, K]
    torch.cuda.synchronize()
    dyo, wto = oracle.quantize(oracle_input(dy)), oracle.quantize_transposed(oracle_input(w))
    dyto, ato = oracle.quantize_transposed(oracle_input(dy)), oracle.quantize_transposed(oracle_input(a))
    for g, o, lbl in ((dyq, dyo, "dY"), (wtq, wto, "W^T"), (dytq, dyto, "dY^T"), (atq, ato, "A^T")):
        assert_quant_equal(g, o, lbl)
    ref, tot = oracle.gemm_ref(*dyo, *wto)
    check_gemm_bound(c_to_f64(dx), ref, tot, False, "dX %dx%dx%d" % (M, K, N))
    ref, tot = oracle.gemm_ref(*dyto, *ato)
    check_gemm_bound(c_to_f64(dw), ref, tot, True, "dW %dx%dx%d" % (N, K, M))


def test_backward_gemms_config3_full_size_sampled():
    """The FFN up-projection's dgrad (16384 x 3072, contracting 14336) and wgrad
    (14336 x 3072, contracting 16384) on the fast GEMM path; sampled rows and
    columns of every output tile against the oracle."""
    nv = _nv()
    a, w, dy = workloads.activations(3), workloads.weights(3), workloads.output_grads(3)
    log("cfg3 backward: dY", tuple(dy.shape))
    ad, wd, dyd = a.to(dev()), w.to(dev()), dy.to(dev())
    dx = nv.gemm(nv.quantize(dyd), nv.quantize_transposed(wd))
    dw = nv.gemm(nv.quantize_transposed(dyd), nv.quantize_transposed(ad))
    torch.cuda.synchronize()
    dyo, wto = oracle.quantize(oracle_input(dy)), oracle.quantize_transposed(oracle_input(w))
    for c, (ao, bo), lbl in ((dx, (dyo, wto), "dX"),
                             (dw, (oracle.quantize_transposed(oracle_input(dy)),
                                   oracle.quantize_transposed(oracle_input(a))), "dW")):
        check_gemm_tiles(c_to_f64(c), ao, bo, True, "cfg3 " + lbl, seed=len(lbl))
