"""Calls on two streams at once.  The library keeps no state between calls, so
independent calls on different streams (no shared output buffer) must give
exactly what they give one after the other: a row-wise quantize and a W4A4
GEMM on one stream, a KV-cache round trip, a transposed quantize and
attention over the packed cache on the other, launched back to back on both
streams and compared bit for bit with the results of the same calls run in
sequence on the default stream."""
import pytest
import torch

from tests.gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def test_calls_on_two_streams_match_sequential():
    nv = _nv()
    gen = torch.Generator().manual_seed(99)
    a = torch.randn(2048, 3072, generator=gen).to(torch.bfloat16).to(dev())
    w = (torch.randn(3072, 3072, generator=gen) * 0.02).to(torch.bfloat16).to(dev())
    kv = torch.randn(8, 4096, 128, generator=gen).to(torch.bfloat16).to(dev())
    dy = (torch.randn(1024, 2048, generator=gen) * 1e-3).to(torch.bfloat16).to(dev())
    q = torch.randn(8, 512, 128, generator=gen).to(torch.bfloat16).to(dev())
    wq = nv.quantize(w)
    torch.cuda.synchronize()

    def linear():
        aq = nv.quantize(a)
        return list(aq) + [nv.gemm(aq, wq)]

    def cache_and_backward():
        kq = nv.kv_quantize(kv)
        return list(kq) + [nv.kv_dequantize(*kq)] + list(nv.quantize_transposed(dy)) + [nv.kv_attention(q, kq, kq)]

    want_a, want_b = linear(), cache_and_backward()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(3):
        log("two streams, repetition", rep)
        with torch.cuda.stream(s1):
            got_a = linear()
        with torch.cuda.stream(s2):
            got_b = cache_and_backward()
        torch.cuda.synchronize()
        for name, got, want in (("linear", got_a, want_a), ("cache/backward", got_b, want_b)):
            for i, (g, x) in enumerate(zip(got, want)):
                assert torch.equal(g, x), "%s output %d differs on repetition %d" % (name, i, rep)
