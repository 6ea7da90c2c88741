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
