"""GPU parity of the W4A4 GEMM with the oracle's fp64 reference:
max |C - ref| <= 1e-5 * sum_k |a_k b_k| per output element (plus half a bf16
ulp of C when the output is bf16), on small ragged shapes and on sampled
rows/columns of the four linear workloads at full size."""
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


def _rand(shape, seed, dtype=torch.bfloat16):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=gen) * torch.exp(0.5 * torch.randn(1, shape[1], generator=gen))
    return x.to(dtype)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (5, 7, 48), (256, 256, 256), (300, 200, 128), (257, 513, 80),
                                   (130, 70, 3072), (512, 768, 640), (300, 200, 512), (1000, 1004, 768),
                                   (17, 516, 1024), (513, 4, 256)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_small_ragged(M, N, K, out):
    log("gemm", M, N, K, out)
    nv = _nv()
    a = _rand((M, K), M * 31 + K)
    b = _rand((N, K), N * 17 + K + 1)
    aq = nv.quantize(a.to(dev()))
    bq = nv.quantize(b.to(dev()))
    c = nv.gemm(aq, bq, out_dtype=out)
    ao = oracle.quantize(oracle_input(a))
    bo = oracle.quantize(oracle_input(b))
    assert_quant_equal(aq, ao, "A")
    assert_quant_equal(bq, bo, "B")
    ref, tot = oracle.gemm_ref(*ao, *bo)
    check_gemm_bound(c_to_f64(c), ref, tot, out == torch.bfloat16, "gemm %dx%dx%d" % (M, N, K))
    if out == torch.bfloat16:
        c32 = nv.gemm(aq, bq, out_dtype=torch.float32)
        assert torch.equal(c32.to(torch.bfloat16), c)  # bf16 output = RN_bf16(fp32 output)


def test_gemm_unit_scales_exact():
    """Scales 1.0 and s_g = 1: every partial sum is a small dyadic, so the
    MFMA result must equal the exact numpy matmul."""
    nv = _nv()
    rng = np.random.default_rng(7)
    M, N, K = 256, 512, 512
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = np.full((M, K // 16), 0x38, np.uint8)
    sb = np.full((N, K // 16), 0x38, np.uint8)
    one = torch.ones(1, device=dev())
    t = lambda a: torch.from_numpy(a).to(dev())
    c = nv.gemm((t(ac), t(sa), one), (t(bc), t(sb), one), out_dtype=torch.float32)
    ref, _ = oracle.gemm_ref(ac, sa, 1.0, bc, sb, 1.0)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_gemm_config_full_size(cfg):
    nv = _nv()
    c_ = workloads.CONFIGS[cfg]
    a = workloads.activations(cfg)
    w = workloads.weights(cfg)
    log("config", cfg, "A", tuple(a.shape), "W", tuple(w.shape))
    ad, wd = a.to(dev()), w.to(dev())
    wq = nv.quantize(wd)
    out = torch.float32 if c_["c_dtype"] == "f32" else torch.bfloat16
    if cfg == 3:
        c, aq = nv.gemm_fused_act(ad, wq, out_dtype=out)
    else:
        aq = nv.quantize(ad)
        c = nv.gemm(aq, wq, out_dtype=out)
    torch.cuda.synchronize()
    ao = oracle.quantize(oracle_input(a))
    wo = oracle.quantize(oracle_input(w))
    assert_quant_equal(aq, ao, "cfg%d A" % cfg)
    assert_quant_equal(wq, wo, "cfg%d W" % cfg)
    check_gemm_tiles(c_to_f64(c), ao, wo, out == torch.bfloat16, "cfg%d" % cfg, seed=cfg)
    if cfg == 3:  # the fused call equals quantize + gemm bit for bit
        c2 = nv.gemm(nv.quantize(ad), wq, out_dtype=out)
        assert torch.equal(c, c2)


def test_gemm_deterministic():
    nv = _nv()
    a = nv.quantize(_rand((1024, 1024), 1).to(dev()))
    b = nv.quantize(_rand((768, 1024), 2).to(dev()))
    assert torch.equal(nv.gemm(a, b), nv.gemm(a, b))


def test_gemm_many_tiles_with_ragged_edges():
    """More tiles than workgroups (each walks several tiles), last tile row and
    column ragged; every output tile sampled against the oracle."""
    nv = _nv()
    M, N, K = 16 * 256 + 100, 17 * 256 - 60, 512
    log("gemm many tiles", M, N, K)
    a = _rand((M, K), 11)
    b = _rand((N, K), 12)
    aq, bq = nv.quantize(a.to(dev())), nv.quantize(b.to(dev()))
    c = c_to_f64(nv.gemm(aq, bq, out_dtype=torch.bfloat16))
    ao, bo = oracle.quantize(oracle_input(a)), oracle.quantize(oracle_input(b))
    check_gemm_tiles(c, ao, bo, True, "many tiles")


@pytest.mark.parametrize("K", [48, 512, 1024])
def test_gemm_every_scale_byte(K):
    """Every finite E4M3 scale byte (0x00..0x7E, subnormals included) on both
    operands, random codes, s_g = 1: within the bound of the fp64 reference.
    K = 48 runs the general kernel, K % 512 == 0 the direct-to-LDS one."""
    nv = _nv()
    rng = np.random.default_rng(K)
    M, N = 260, 264
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    m_i, kb_i = np.meshgrid(np.arange(M), np.arange(K // 16), indexing="ij")
    sa = ((m_i + 7 * kb_i) % 127).astype(np.uint8)
    n_i, kb_j = np.meshgrid(np.arange(N), np.arange(K // 16), indexing="ij")
    sb = ((3 * n_i + 5 * kb_j + 11) % 127).astype(np.uint8)
    assert set(np.unique(sa)) == set(range(127)) and set(np.unique(sb)) == set(range(127))
    one = torch.ones(1, device=dev())
    t = lambda a: torch.from_numpy(a).to(dev())
    c = nv.gemm((t(ac), t(sa), one), (t(bc), t(sb), one), out_dtype=torch.float32)
    ref, tot = oracle.gemm_ref(ac, sa, 1.0, bc, sb, 1.0)
    check_gemm_bound(c_to_f64(c), ref, tot, False, "every scale byte K=%d" % K)


def test_fused_act_given_scale_matches_computed():
    """nvfp4_gemm_fused_act with the activation scale given (NVFP4_SCALE_GIVEN, written
    beforehand on the stream by nvfp4_global_scale) equals the computed-scale call bit for
    bit: packed activation, scale and C; and equals quantize + gemm with that scale."""
    nv = _nv()
    for cfg, M in ((3, 2048), (2, 1000)):
        a = workloads.activations(cfg, M=M).to(dev())
        wq = nv.quantize(workloads.weights(cfg, N=520).to(dev()))
        c1, q1 = nv.gemm_fused_act(a, wq)
        sg = nv.global_scale(a)
        c2, q2 = nv.gemm_fused_act(a, wq, s_g=sg)
        c3 = nv.gemm(nv.quantize(a, s_g=sg), wq)
        torch.cuda.synchronize()
        log("fused_act given scale, cfg", cfg, "M", M)
        assert q2[2] is sg
        for u, v in zip(q1, q2):
            assert torch.equal(u, v)
        assert torch.equal(c1, c2) and torch.equal(c2, c3)
        # a different given scale is used as given (saturating codes), not recomputed
        half = sg * 0.5
        c4, q4 = nv.gemm_fused_act(a, wq, s_g=half)
        ref = nv.quantize(a, s_g=half)
        torch.cuda.synchronize()
        assert torch.equal(q4[0], ref[0]) and torch.equal(q4[1], ref[1]) and torch.equal(c4, nv.gemm(ref, wq))


def _fast_tile_cols(M, N, cus=256):
    """Output columns per tile the fast path takes (its launcher's rule on a 256-CU device):
    256, or 192 when 256 x 192 tiles need fewer rounds of the persistent grid (a round of them
    counting 0.87 of a 256 x 256 round)."""
    tm = (M + 255) // 256
    r256 = (tm * ((N + 255) // 256) + cus - 1) // cus
    r192 = (tm * ((N + 191) // 192) + cus - 1) // cus
    return 192 if r192 * 0.87 < r256 else 256


@pytest.mark.parametrize("M,N,K,cols", [(512, 384, 512, 192), (520, 400, 1024, 192), (4096, 4096, 512, 256),
                                        (4000, 4000, 512, 256), (4096, 3072, 512, 192)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_fast_tile_shapes(M, N, K, cols, out):
    """Both output tiles of the direct-to-LDS kernel, 256 x 256 and 256 x 192, with full tiles
    (the staged bf16 epilogue, whole and shared 128-byte lines) and ragged last tiles."""
    assert _fast_tile_cols(M, N) == cols
    log("gemm fast tiles", M, N, K, "tile cols", cols, out)
    nv = _nv()
    a = _rand((M, K), M + 3 * N)
    b = _rand((N, K), N + 5 * M)
    aq, bq = nv.quantize(a.to(dev())), nv.quantize(b.to(dev()))
    c = nv.gemm(aq, bq, out_dtype=out)
    ao, bo = oracle.quantize(oracle_input(a)), oracle.quantize(oracle_input(b))
    if M * N <= 600 * 600:
        ref, tot = oracle.gemm_ref(*ao, *bo)
        check_gemm_bound(c_to_f64(c), ref, tot, out == torch.bfloat16, "fast tiles %dx%dx%d" % (M, N, K))
    else:
        check_gemm_tiles(c_to_f64(c), ao, bo, out == torch.bfloat16, "fast tiles %dx%dx%d" % (M, N, K), tile=128)
    if out == torch.bfloat16:
        assert torch.equal(nv.gemm(aq, bq, out_dtype=torch.float32).to(torch.bfloat16), c)
