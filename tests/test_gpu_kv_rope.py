"""GPU parity of kv_rope_quantize_append (RoPE of new keys fused into the NVFP4
KV append) with the oracle's fp64 rotation followed by its exact quantizer
under the cache's frozen head scales.

The kernel forms and reduces the angle in fp64 and rotates in fp32: its cos
and sin are within 2^-21.6 of the exact values (the reduced angle rounded to
fp32, at most 2^-24 pi, plus sincosf's error) and the two products and the fma
add 2^-23 relative, so each rotated element is within
  tau = 4 * (|x_2i| + |x_2i+1|) * 2^-21
of the exact one.  Codes and scale bytes may differ from the oracle's only
where the exact value lies within tau of a decision boundary."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import check_quant_near_exact, dev, log

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _tau(bits):
    x = np.abs((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    pair = x[..., 0::2] + x[..., 1::2]
    return 4 * np.repeat(pair, 2, axis=-1) * 2.0 ** -21


def _run(H, Tc, Tn, D, off, positions, base, seed, label):
    nv = _nv()
    k0, _ = workloads.kv_cache(H, Tc, D, sinks=min(4, Tc))
    gen = torch.Generator().manual_seed(seed)
    k_new = (torch.randn(H, Tn, D, generator=gen) * 1.5).to(torch.bfloat16)
    cache = nv.kv_quantize(k0.to(dev()))
    before = [t.clone() for t in cache]
    pos_t = None if positions is None else torch.tensor(positions, dtype=torch.int32, device=dev())
    nv.kv_rope_quantize_append(k_new.to(dev()), cache, off, positions=pos_t, base=base)
    torch.cuda.synchronize()
    codes, scales, hs = cache
    rows = slice(off, off + Tn)
    for t, b in zip(cache[:2], before[:2]):  # every byte outside the appended rows is unchanged
        t_c, b_c = t.clone(), b.clone()
        t_c[:, rows] = 0
        b_c[:, rows] = 0
        assert torch.equal(t_c, b_c)
    assert torch.equal(hs, before[2])
    bits = workloads.bf16_bits(k_new)
    pos = np.arange(off, off + Tn) if positions is None else np.asarray(positions)
    y = oracle.rope(bits, pos, base)
    tau = _tau(bits)
    hsn = hs.cpu().numpy()
    for h in range(H):
        check_quant_near_exact(codes[h, rows], scales[h, rows], y[h], tau[h], hsn[h], "%s head %d" % (label, h))


@pytest.mark.parametrize("H,Tc,Tn,D,off,explicit,base", [
    (2, 256, 64, 128, 100, False, 10000.0), (3, 300, 37, 64, 0, True, 10000.0), (1, 64, 64, 16, 0, False, 500.0),
    (2, 512, 200, 256, 311, True, 10000.0), (1, 80, 1, 128, 79, False, 10000.0),
    (1, 16, 5, 2048, 3, False, 10000.0), (2, 40, 33, 32, 1, True, 10000.0)])  # largest head_dim; 32
def test_rope_append(H, Tc, Tn, D, off, explicit, base):
    log("rope append", H, Tc, Tn, D, off, explicit, base)
    positions = None
    if explicit:  # positions far past the cache length: the fp64 angle reduction matters
        positions = np.random.default_rng(Tn).integers(0, 70000, Tn).astype(np.int32).tolist()
    _run(H, Tc, Tn, D, off, positions, base, seed=H * 17 + Tn, label="rope %dx%d/%d" % (H, Tn, D))


def test_rope_at_position_zero_equals_plain_append():
    """p = 0 is the identity: the rotated append must equal kv_quantize_append bit for bit."""
    nv = _nv()
    k0, _ = workloads.kv_cache(2, 128, 128)
    k_new = k0[:, :50].contiguous().flip(1).contiguous().to(dev())
    a = nv.kv_quantize(k0.to(dev()))
    b = tuple(t.clone() for t in a)
    nv.kv_rope_quantize_append(k_new, a, 30, positions=torch.zeros(50, dtype=torch.int32, device=dev()))
    nv.kv_quantize_append(k_new, b, 30)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_rope_append_full_cache_tail():
    """24 heads: 4096 new keys rotated into rows 61440 .. 65535 of a 65,536-token cache."""
    log("rope append 24 x 4096 into 65536")
    _run(24, 65536, 4096, 128, 61440, None, 10000.0, seed=5, label="full")


def test_rope_append_empty():
    nv = _nv()
    k0, _ = workloads.kv_cache(2, 64, 128)
    a = nv.kv_quantize(k0.to(dev()))
    b = tuple(t.clone() for t in a)
    nv.kv_rope_quantize_append(torch.empty(2, 0, 128, dtype=torch.bfloat16, device=dev()), a, 64)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
