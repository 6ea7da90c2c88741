"""GPU parity of the NVFP4 KV cache (kv_quantize / kv_dequantize) with the
oracle: codes, scale bytes, per-head scales and the bf16 round trip bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import dev, f32_bits, log

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _check(kv_cpu, label):
    nv = _nv()
    kv = kv_cpu.to(dev())
    codes, scales, hs = nv.kv_quantize(kv)
    out = nv.kv_dequantize(codes, scales, hs)
    torch.cuda.synchronize()
    oc, os_, oh = oracle.kv_quantize(workloads.bf16_bits(kv_cpu))
    assert np.array_equal(f32_bits(hs.cpu().numpy()), f32_bits(oh)), label + ": head scales"
    gs = scales.cpu().numpy()
    assert np.array_equal(gs, os_), "%s: %d scale bytes differ" % (label, (gs != os_).sum())
    gc = codes.cpu().numpy()
    assert np.array_equal(gc, oc), "%s: %d code bytes differ" % (label, (gc != oc).sum())
    want = oracle.kv_dequantize(oc, os_, oh)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want), "%s: %d dequantized values differ" % (label, (got != want).sum())


@pytest.mark.parametrize("H,T,D", [(1, 1, 16), (3, 5, 32), (24, 100, 128), (2, 333, 64)])
def test_kv_small(H, T, D):
    log("kv", H, T, D)
    k, v = workloads.kv_cache(H, T, D, sinks=min(4, T))
    _check(k, "K %dx%dx%d" % (H, T, D))
    _check(v, "V %dx%dx%d" % (H, T, D))


def test_kv_empty_tokens():
    nv = _nv()
    kv = torch.zeros(4, 0, 128, dtype=torch.bfloat16, device=dev())
    codes, scales, hs = nv.kv_quantize(kv)
    assert hs.cpu().tolist() == [0.0] * 4
    assert nv.kv_dequantize(codes, scales, hs).shape == (4, 0, 128)


def test_kv_full_size():
    k, v = workloads.kv_cache()
    log("kv full", tuple(k.shape))
    _check(k, "K full")
    _check(v, "V full")


@pytest.mark.parametrize("H,T,D,offset,t_new", [(4, 256, 128, 100, 48), (3, 64, 64, 63, 1), (24, 512, 128, 448, 64)])
def test_kv_append_in_place(H, T, D, offset, t_new):
    """A cache filled by kv_quantize, then new tokens appended at an offset with
    the frozen head scales (some of them beyond the scale's range, which
    saturate): the appended rows equal the oracle's quantization of the new
    tokens under those scales, every other byte of the cache is unchanged."""
    nv = _nv()
    log("kv append", H, T, D, offset, t_new)
    k0, _ = workloads.kv_cache(H, T, D, sinks=4)
    gen = torch.Generator().manual_seed(H * 1000 + offset)
    new = torch.randn(H, t_new, D, generator=gen)
    new[:, 0, :3] *= 40.0  # beyond 2688 * s_g of the frozen scale: saturates
    new = new.to(torch.bfloat16)
    cache = nv.kv_quantize(k0.to(dev()))
    before = [t.cpu().numpy().copy() for t in cache]
    nv.kv_quantize_append(new.to(dev()), cache, offset)
    torch.cuda.synchronize()
    hs = before[2]
    want_c, want_s = before[0].copy(), before[1].copy()
    nb = workloads.bf16_bits(new)
    for h in range(H):
        oc, os_, _ = oracle.quantize(np.ascontiguousarray(nb[h]), s_g=np.float32(hs[h]))
        want_c[h, offset:offset + t_new] = oc
        want_s[h, offset:offset + t_new] = os_
    got_c, got_s = cache[0].cpu().numpy(), cache[1].cpu().numpy()
    assert np.array_equal(f32_bits(cache[2].cpu().numpy()), f32_bits(hs)), "head scales must not change"
    assert np.array_equal(got_s, want_s), "%d scale bytes differ" % (got_s != want_s).sum()
    assert np.array_equal(got_c, want_c), "%d code bytes differ" % (got_c != want_c).sum()
    assert (want_s[:, offset] == 0x7E).any(), "the test should exercise saturation"
