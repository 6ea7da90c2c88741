"""Seeded random sweep of the library against the oracle, beyond the fixed
shapes of the other parity tests: each case draws its sizes, input dtype,
scale mode (computed, or given at a random multiple of the computed one so
that some blocks saturate), FourOverSix on or off, and a value mix
(heavy-tailed columns, sparse outliers, zeros with signed zeros, a tiny
tensor whose s_g takes the exact slow path, or values on the NVFP4 grid,
where every rounding is a tie).  Quantize, quantize along rows and dequantize
must equal the oracle bit for bit, as must the KV-cache calls; the GEMM
(the fast kernel or the general one, by shape) must stay within
1e-5 * sum|a b| (+ half a bf16 ulp) of the fp64 reference everywhere.
Attention, the adaLN-fused quantizer and the RoPE-fused append are swept
through the checks of their own parity tests."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import assert_quant_equal, c_to_f64, check_gemm_bound, dev, f32_bits, log, oracle_input

pytestmark = pytest.mark.gpu

KINDS = ("normal", "lognormal_cols", "outliers", "zeros", "tiny", "grid")


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _values(rng, rows, cols, kind):
    """float32 [rows, cols] of the given mix; every value is exact in bf16 except in "normal" etc.,
    which the caller rounds to its dtype."""
    if kind == "normal":
        x = rng.standard_normal((rows, cols))
    elif kind == "lognormal_cols":
        x = rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((1, cols)))
    elif kind == "outliers":
        x = rng.standard_normal((rows, cols))
        x[rng.random((rows, cols)) < 0.01] *= 50.0
    elif kind == "zeros":
        x = rng.standard_normal((rows, cols))
        x[rng.random((rows, cols)) < 0.3] = 0.0
        x[rng.random((rows, cols)) < 0.05] = -0.0
    elif kind == "tiny":
        x = rng.standard_normal((rows, cols)) * 1e-31
    else:  # grid: val(code) * val(scale byte) * 2^-7, exact in bf16 (<= 5 significant bits)
        mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        sv = np.array([oracle.e4m3_value(int(b)) for b in range(127)])
        sc = rng.integers(1, 127, (rows, (cols + 15) // 16))
        q = mags[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
        x = q * np.repeat(sv[sc], 16, axis=1)[:, :cols] * 2.0 ** -7
    return torch.from_numpy(np.asarray(x, np.float32))


def _draw(case, rows_max, k_max):
    rng = np.random.default_rng(7000 + case)
    rows = 16 * int(rng.integers(1, rows_max // 16 + 1))
    k = 16 * int(rng.integers(1, k_max // 16 + 1))
    dtype = (torch.float32, torch.bfloat16)[case % 2]
    kind = KINDS[case % len(KINDS)]
    given = bool((case // 2) % 2)
    k46 = bool((case // 4) % 2)
    return rng, rows, k, dtype, kind, given, k46


@pytest.mark.parametrize("case", range(48))
def test_fuzz_quantize_transposed_dequantize(case):
    nv = _nv()
    rng, rows, k, dtype, kind, given, k46 = _draw(case, 640, 2048)
    log("fuzz quantize", case, rows, k, dtype, kind, "given" if given else "computed", "4o6" if k46 else "")
    x_cpu = _values(rng, rows, k, kind).to(dtype)
    xo = oracle_input(x_cpu)
    x = x_cpu.to(dev())
    s_g = None
    if given:
        s_g = np.float32(oracle.global_scale(oracle.amax(xo)) * float(rng.choice([0.25, 0.7, 1.0, 3.0])))
    s_dev = None if s_g is None else torch.tensor([s_g], dtype=torch.float32, device=dev())
    g = nv.quantize(x, s_g=s_dev, four_over_six=k46)
    gt = nv.quantize_transposed(x, s_g=s_dev, four_over_six=k46)
    torch.cuda.synchronize()
    o = oracle.quantize(xo, s_g=s_g, four_over_six=k46)
    assert_quant_equal(g, o, "case %d row-wise" % case)
    assert_quant_equal(gt, oracle.quantize_transposed(xo, s_g=s_g, four_over_six=k46), "case %d along rows" % case)
    for out in ("bf16", "f32"):
        y = nv.dequantize(g[0], g[1], g[2], dtype=torch.bfloat16 if out == "bf16" else torch.float32).cpu()
        want = oracle.dequantize(o[0], o[1], o[2], out)
        got = y.view(torch.int16).numpy().view(np.uint16) if out == "bf16" else f32_bits(y.numpy())
        assert np.array_equal(got, want if out == "bf16" else f32_bits(want)), "case %d dequantize %s" % (case, out)


@pytest.mark.parametrize("case", range(24))
def test_fuzz_gemm(case):
    nv = _nv()
    rng = np.random.default_rng(9000 + case)
    M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
    if case % 3 == 0:  # shapes the fast kernel takes: K % 512 == 0, N % 4 == 0
        K = 512 * int(rng.integers(1, 4))
        N = 4 * max(1, N // 4)
    else:
        K = 16 * int(rng.integers(1, 96))
    out = (torch.float32, torch.bfloat16)[case % 2]
    kind_a, kind_b = KINDS[case % 4], KINDS[(case + 1) % 4]
    log("fuzz gemm", case, M, N, K, out, kind_a, kind_b)
    a = _values(rng, M, K, kind_a).to(torch.bfloat16)
    b = (_values(rng, N, K, kind_b) * 0.05).to(torch.bfloat16)
    aq, bq = nv.quantize(a.to(dev())), nv.quantize(b.to(dev()))
    c = nv.gemm(aq, bq, out_dtype=out)
    torch.cuda.synchronize()
    ao, bo = oracle.quantize(oracle_input(a)), oracle.quantize(oracle_input(b))
    assert_quant_equal(aq, ao, "case %d A" % case)
    assert_quant_equal(bq, bo, "case %d B" % case)
    ref, tot = oracle.gemm_ref(*ao, *bo)
    check_gemm_bound(c_to_f64(c), ref, tot, out == torch.bfloat16, "case %d gemm %dx%dx%d" % (case, M, N, K))


@pytest.mark.parametrize("case", range(12))
def test_fuzz_kv(case):
    nv = _nv()
    rng = np.random.default_rng(11000 + case)
    H, T, D = int(rng.integers(1, 6)), int(rng.integers(1, 700)), 16 * int(rng.integers(1, 17))
    k46 = bool(case % 2)
    kind = KINDS[case % len(KINDS)]
    log("fuzz kv", case, H, T, D, kind, "4o6" if k46 else "")
    kv_cpu = _values(rng, H * T, D, kind).reshape(H, T, D).to(torch.bfloat16)
    codes, scales, hs = nv.kv_quantize(kv_cpu.to(dev()), four_over_six=k46)
    deq = nv.kv_dequantize(codes, scales, hs)
    torch.cuda.synchronize()
    oc, os_, oh = oracle.kv_quantize(workloads.bf16_bits(kv_cpu), four_over_six=k46)
    assert np.array_equal(f32_bits(hs.cpu().numpy()), f32_bits(oh)), "case %d head scales" % case
    assert np.array_equal(scales.cpu().numpy(), os_), "case %d scale bytes" % case
    assert np.array_equal(codes.cpu().numpy(), oc), "case %d codes" % case
    got = deq.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, oracle.kv_dequantize(oc, os_, oh)), "case %d round trip" % case


@pytest.mark.parametrize("case", range(10))
def test_fuzz_attention(case):
    """Random head counts, query and cache lengths, attended prefixes, query scales, softmax
    factors (negative and zero included) and workspaces, within the bound of the attention tests
    (which also checks that the bound stays below |ref| for most elements)."""
    from tests.test_gpu_attention import _run as attention_run
    rng = np.random.default_rng(13000 + case)
    H, Tq, Tc = int(rng.integers(1, 4)), int(rng.integers(1, 400)), int(rng.integers(1, 3000))
    T = int(rng.integers(1, Tc + 1))
    qscale = float(rng.choice([0.5, 1.0, 3.0]))
    scale = [None, None, -0.15, 0.0, 0.3][case % 5]
    ws = [(None,), (0,), (None, 0)][case % 3]
    log("fuzz attention", case, H, Tq, Tc, T, qscale, scale, ws)
    attention_run(H, Tq, Tc, T, seed=13000 + case, qscale=qscale, scale=scale, workspaces=ws)


@pytest.mark.parametrize("case", range(12))
def test_fuzz_adaln(case):
    """Random row counts, widths, group sizes, eps and input dtypes for the adaLN-fused
    quantizer, against fp64 adaLN + exact quantization with the near-boundary criterion of its
    parity tests (both the given and the computed scale)."""
    from tests.test_gpu_adaln import _run as adaln_run
    rng = np.random.default_rng(15000 + case)
    rows, k = int(rng.integers(1, 600)), 16 * int(rng.integers(1, 257))
    rpg = int(rng.integers(1, rows + 50))
    eps = float(rng.choice([1e-6, 1e-5, 1.0]))
    dtype = (torch.bfloat16, torch.float32)[case % 2]
    gen = torch.Generator().manual_seed(15000 + case)
    x = torch.randn(rows, k, generator=gen) * torch.exp(torch.randn(1, k, generator=gen)) + \
        torch.randn(rows, 1, generator=gen) * float(rng.choice([0.0, 1.0, 10.0]))
    G = (rows + rpg - 1) // rpg
    shift = torch.randn(G, k, generator=gen) * float(rng.choice([0.0, 0.3, 2.0]))
    scale = torch.randn(G, k, generator=gen) * float(rng.choice([0.0, 0.3, 1.0]))
    log("fuzz adaln", case, rows, k, rpg, eps, dtype)
    adaln_run(x.to(dtype), shift, scale, rpg, eps, "fuzz %d" % case)


@pytest.mark.parametrize("case", range(10))
def test_fuzz_rope_append(case):
    """Random head counts, head sizes (every one the kernel takes), cache lengths, offsets,
    explicit or implicit positions and bases for the RoPE-fused append, against fp64 RoPE +
    exact quantization with the near-boundary criterion of its parity tests; bytes outside the
    appended rows must not change."""
    from tests.test_gpu_kv_rope import _run as rope_run
    rng = np.random.default_rng(17000 + case)
    H = int(rng.integers(1, 5))
    D = int(rng.choice([16, 32, 64, 128, 256, 512, 1024, 2048]))
    Tc = int(rng.integers(1, 600 if D <= 256 else 80))
    Tn = int(rng.integers(1, Tc + 1))
    off = int(rng.integers(0, Tc - Tn + 1))
    positions = rng.integers(0, 100000, Tn).astype(np.int32).tolist() if case % 2 else None
    base = float(rng.choice([500.0, 10000.0, 1e6]))
    log("fuzz rope", case, H, Tc, Tn, D, off, positions is not None, base)
    rope_run(H, Tc, Tn, D, off, positions, base, seed=17000 + case, label="fuzz %d" % case)
