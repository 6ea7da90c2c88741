"""GPU parity of nvfp4_quantize / nvfp4_dequantize with the CPU oracle:
codes, scale bytes, s_g and dequantized values bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_quant_equal, dev, log, oracle_input

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _quant_both(x_cpu, label, s_g=None):
    nv = _nv()
    x = x_cpu.to(dev())
    if s_g is None:
        g = nv.quantize(x)
        o = oracle.quantize(oracle_input(x_cpu))
    else:
        g = nv.quantize(x, s_g=torch.tensor([s_g], dtype=torch.float32, device=dev()))
        o = oracle.quantize(oracle_input(x_cpu), s_g=np.float32(s_g))
    torch.cuda.synchronize()
    assert_quant_equal(g, o, label)
    return g, o


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,k", [(1, 16), (3, 48), (7, 80), (33, 272), (129, 3072), (1000, 1024)])
def test_quantize_random(dtype, rows, k):
    log("quantize random", dtype, rows, k)
    gen = torch.Generator().manual_seed(rows * 7919 + k)
    x = torch.randn(rows, k, generator=gen) * torch.exp(torch.randn(1, k, generator=gen))
    x[torch.rand(rows, k, generator=gen) < 0.01] *= 30
    _quant_both(x.to(dtype), "random %s %dx%d" % (dtype, rows, k))


def test_quantize_on_grid_and_ties():
    """Inputs on the quantization grid and exactly on E2M1/E4M3 midpoints: every
    element takes the exact tie-resolution path."""
    log("quantize on-grid / ties")
    rng = np.random.default_rng(5)
    rows, k = 64, 256
    s_g = np.float32(2.0 ** -7)
    scales = rng.integers(1, 127, (rows, k // 16))
    scales[0, 0] = 0x7E  # the tensor maximum 6 * 448 * s_g fixes s_g = 2^-7
    sv = np.array([oracle.e4m3_value(int(b)) for b in range(127)])[scales.astype(int)]
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5])
    q = mags[rng.integers(0, len(mags), (rows, k))] * rng.choice([-1, 1], (rows, k))
    for b in range(k // 16):  # a +-6 in every block pins its scale to the chosen byte
        q[np.arange(rows), 16 * b + rng.integers(0, 16, rows)] = 6.0 * rng.choice([-1, 1], rows)
    q[0, 0] = 6.0
    x = (q * np.repeat(sv, 16, axis=1) * float(s_g)).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), q * np.repeat(sv, 16, axis=1) * float(s_g))
    _quant_both(torch.from_numpy(x), "on-grid f32")
    _quant_both(torch.from_numpy(x).to(torch.bfloat16), "on-grid bf16")


def test_quantize_block_scale_ties():
    log("quantize E4M3 ties")
    s_g = 2.0 ** -10
    vals = [oracle.e4m3_value(b) for b in range(127)]
    rows = []
    for i in range(126):
        mid = 0.5 * (vals[i] + vals[i + 1]) * 6 * s_g
        rows.append([mid] + [mid * j / 17.0 for j in range(15)])
    x = torch.tensor(rows, dtype=torch.float32)
    x[0, 1] = 2688 * s_g
    _quant_both(x, "e4m3 ties f32")


def test_quantize_zero_tiny_and_signed_zero():
    log("quantize zero / tiny / -0")
    z = torch.zeros(4, 64)
    z[1, 5] = -0.0
    z[2, 7] = -0.0
    _quant_both(z, "all zero f32")
    _quant_both(z.to(torch.bfloat16), "all zero bf16")
    gen = torch.Generator().manual_seed(3)
    tiny = torch.randn(8, 64, generator=gen) * 1e-33  # s_g below 2^-100: exact slow path
    _quant_both(tiny, "tiny f32")
    under = torch.randn(8, 64, generator=gen)
    under[3] *= 1e-6  # blocks whose scale underflows to E4M3 zero or subnormal
    under[4] *= 1e-4
    under[5, 16:32] = -1e-9
    _quant_both(under, "underflow blocks")
    _quant_both(torch.zeros(0, 32), "empty")


def test_quantize_given_scale_saturates():
    log("quantize given scale")
    gen = torch.Generator().manual_seed(4)
    x = torch.randn(16, 128, generator=gen)
    _quant_both(x, "given scale (saturating)", s_g=float(np.float32(0.3 / 2688)))
    _quant_both(x, "given scale (loose)", s_g=float(np.float32(100.0 / 2688)))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_random_and_hazards(dtype):
    log("dequantize", dtype)
    nv = _nv()
    rng = np.random.default_rng(6)
    rows, k = 97, 512
    codes = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 127, (rows, k // 16), dtype=np.uint8)
    # s_g values chosen so that some fp32 products land exactly on bf16 midpoints
    for s_g in [np.float32(1.0), np.float32(0.0123), np.float32((2 ** 23 + 2 ** 15 + 1) / 2 ** 23 / 1.5),
                np.float32(1.17e-36), np.float32(3e34)]:
        y = nv.dequantize(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                          torch.tensor([s_g], device=dev()), dtype=dtype)
        want = oracle.dequantize(codes, scales, s_g, "bf16" if dtype == torch.bfloat16 else "f32")
        got = y.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else y.cpu().numpy()
        if dtype == torch.bfloat16:
            assert np.array_equal(got, want), "s_g=%r: %d bf16 values differ" % (s_g, (got != want).sum())
        else:
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "s_g=%r" % s_g


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_quantize_config_tensors_full_size(cfg):
    """Activations and weights of each linear workload at full size, bit-exact."""
    a = workloads.activations(cfg)
    log("config", cfg, "activations", tuple(a.shape), a.dtype)
    _quant_both(a, "cfg%d A" % cfg)
    w = workloads.weights(cfg)
    log("config", cfg, "weights", tuple(w.shape), w.dtype)
    g, o = _quant_both(w, "cfg%d W" % cfg)
    # dequantized weights, bit-exact
    nv = _nv()
    y = nv.dequantize(g[0], g[1], g[2]).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, oracle.dequantize(o[0], o[1], o[2], "bf16"))


def test_quantize_fp32_multi_pass():
    """An fp32 tensor of more blocks than one pass of the encode grid covers (64
    workgroups per CU, one fp32 block per lane: 67.1M elements on 256 CUs), with a
    ragged last chunk: bit-exact codes and scales, and the fp32 dequantization."""
    rows, k = 8192, 8208  # 67,239,936 elements
    log("quantize fp32 multi-pass", rows, k)
    gen = torch.Generator().manual_seed(8208)
    x = torch.randn(rows, k, generator=gen)
    g, o = _quant_both(x, "fp32 %dx%d" % (rows, k))
    y = _nv().dequantize(g[0], g[1], g[2], dtype=torch.float32).cpu().numpy()
    want = oracle.dequantize(o[0], o[1], o[2], "f32")
    assert np.array_equal(y.view(np.uint32), np.asarray(want).view(np.uint32))


@pytest.mark.parametrize("rows,k,where", [(2048, 8192, "last"), (2048, 8192, "slice3"), (4096, 8192, "first"),
                                           (4096, 8192, "slice15")])
def test_quantize_sliced_amax_outlier(rows, k, where):
    """Tensors large enough for the amax pass to read them in slices (8 and 16 slices
    of 2^18 units here): one outlier at the first or last element or at the first
    element of a slice fixes s_g, and the whole result stays bit-exact."""
    log("quantize sliced amax", rows, k, where)
    gen = torch.Generator().manual_seed(rows + k)
    x = torch.randn(rows, k, generator=gen)
    flat = x.view(-1)
    units = rows * k // 8
    sub = 8 if units == 8 << 18 else 16
    pos = {"last": flat.numel() - 1, "first": 0, "slice3": 3 * (units // sub) * 8,
           "slice15": 15 * (units // sub) * 8}[where]
    flat[pos] = -1000.0
    g, o = _quant_both(x.to(torch.bfloat16), "sliced amax %dx%d %s" % (rows, k, where))
    assert float(g[2].cpu()[0]) == float(np.float32(np.float32(1000.0) / np.float32(2688.0)))


def test_quantize_deterministic():
    nv = _nv()
    a = workloads.activations(2).to(dev())
    r1 = nv.quantize(a)
    r2 = nv.quantize(a)
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


def _global_scale_cases():
    gen = torch.Generator().manual_seed(77)
    yield "f32 3x48", torch.randn(3, 48, generator=gen)
    yield "bf16 1x16", torch.randn(1, 16, generator=gen).to(torch.bfloat16)
    yield "bf16 negative max", (torch.randn(257, 272, generator=gen).abs() * -3.0).to(torch.bfloat16)
    yield "f32 tiny (s_g underflows to subnormal / zero)", torch.full((5, 32), 1e-41)
    yield "f32 zeros", torch.zeros(64, 64)
    yield "bf16 cfg2 activations (outliers)", workloads.activations(2)
    yield "bf16 cfg4 activations", workloads.activations(4)


@pytest.mark.parametrize("case", range(7))
def test_global_scale_matches_oracle_and_quantize(case):
    """nvfp4_global_scale = RN(amax / 2688), bit-exact to the oracle and to
    the s_g that nvfp4_quantize computes; quantizing with it as a given scale
    reproduces the computed-scale result."""
    nv = _nv()
    label, x_cpu = list(_global_scale_cases())[case]
    log("global_scale", label, tuple(x_cpu.shape), x_cpu.dtype)
    x = x_cpu.to(dev())
    g = nv.global_scale(x)
    q = nv.quantize(x)
    qg = nv.quantize(x, s_g=g)
    torch.cuda.synchronize()
    xo = oracle_input(x_cpu)
    want = np.float32(oracle.global_scale(oracle.amax(xo)))
    got = g.cpu().numpy()[0]
    assert got.view(np.uint32) == want.view(np.uint32), "%s: %r != %r" % (label, got, want)
    assert torch.equal(g, q[2])
    for u, v in zip(q[:2], qg[:2]):
        assert torch.equal(u, v)


def test_global_scale_empty_and_reuse():
    """rows == 0 gives s_g = 0; the slot is fully overwritten on every call."""
    nv = _nv()
    s = torch.full((1,), 123.0, device=dev())
    nv.global_scale(torch.empty(0, 32, dtype=torch.bfloat16, device=dev()), out=s)
    torch.cuda.synchronize()
    assert s.item() == 0.0
    x = torch.randn(100, 64, device=dev())
    nv.global_scale(x, out=s)
    a = s.clone()
    nv.global_scale(x * 0.5, out=s)
    nv.global_scale(x, out=s)
    torch.cuda.synchronize()
    assert torch.equal(a, s)
