"""The no-allocation attention entry point (kv_attention_noalloc, for callers
that cannot allocate) through the C ABI, against the existing kv_attention
with a caller workspace of the same size (NVFP4_NOALLOC_SCRATCH_BYTES): bit for
bit, on calls made back to back (a larger input, then a smaller one, so the
second call runs over the first one's leftover scratch contents); and against
the oracle's fp64 attention within the attention tests' bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import c_to_f64, dev, half_ulp_bf16, log

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def _inputs(H, Tq, Tc, seed):
    k, v = workloads.kv_cache(H, Tc, 128, sinks=min(4, Tc))
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, Tq, 128, generator=g).to(torch.bfloat16)
    return q, k, v


def _oracle_check(q, k, v, T, got, q_idx, label):
    ok, ov = oracle.kv_quantize(workloads.bf16_bits(k)), oracle.kv_quantize(workloads.bf16_bits(v))
    ref, wabs, lsum = oracle.kv_attention(workloads.bf16_bits(q), ok, ov, T, 128 ** -0.5, q_idx=q_idx,
                                          return_norm=True)
    H = q.shape[0]
    vf = np.stack([oracle.dequantize(ov[0][h, :T], ov[1][h, :T], ov[2][h], "f32") for h in range(H)])
    vmax = np.abs(vf).max(axis=1)[:, None, :]
    g = c_to_f64(got)[:, q_idx]
    tol = np.maximum(half_ulp_bf16(ref), half_ulp_bf16(g)) + 2.0 ** -9 * wabs + \
        2.0 ** -25 * T * vmax / (lsum[..., None] * (1.0 - 2.0 ** -6))
    worst = float((np.abs(g - ref) / tol).max())
    log(label, "worst err/tol against the oracle %.3g" % worst)
    assert worst <= 1.0


def test_noalloc_attention_matches_workspace_call():
    nv = _nv()
    S = nv.NOALLOC_SCRATCH_BYTES
    # (heads, queries, cache rows, attended rows, seed): the first prefers a split whose partials
    # exceed the scratch (so the split is capped), the second a split that fits, the third is
    # smaller again
    cases = [(24, 1024, 65536, 65536, 41), (4, 256, 20000, 19990, 42), (2, 64, 5000, 4321, 43)]
    want = [nv.kv_attention_workspace_size(H, Tq, T) for H, Tq, _, T, _ in cases]
    log("noalloc: preferred workspaces", want, "scratch", S)
    assert want[0] > S and 0 < want[1] <= S and 0 < want[2] <= S and want[2] < want[1]
    data = []
    for H, Tq, Tc, T, seed in cases:
        q, k, v = _inputs(H, Tq, Tc, seed)
        kq, vq = nv.kv_quantize(k.to(dev())), nv.kv_quantize(v.to(dev()))
        data.append((q, k, v, q.to(dev()), kq, vq, T))
    torch.cuda.synchronize()
    # the no-allocation calls back to back (the second and third over the previous call's scratch),
    # the third one writing into a preallocated output
    outs = []
    for i, (q, k, v, qd, kq, vq, T) in enumerate(data):
        o = torch.full_like(qd, float("nan")) if i == 2 else None
        log("noalloc call", i, tuple(qd.shape), "over", T, "tokens")
        outs.append(nv.kv_attention_noalloc(qd, kq, vq, T, out=o))
        if o is not None:
            assert outs[-1] is o
    torch.cuda.synchronize()
    ws = torch.empty(S, dtype=torch.uint8, device=dev())
    for i, ((q, k, v, qd, kq, vq, T), o) in enumerate(zip(data, outs)):
        ref = nv.kv_attention(qd, kq, vq, T, workspace=ws)
        torch.cuda.synchronize()
        log("noalloc call", i, "equals kv_attention with a %d-byte workspace:" % S, torch.equal(o, ref))
        assert torch.equal(o, ref)
    # and both within the bound of the oracle (sampled queries of the large case)
    for i, (q, k, v, qd, kq, vq, T) in enumerate(data):
        q_idx = np.array([0, 511, 1023]) if i == 0 else np.arange(q.shape[1])
        _oracle_check(q, k, v, T, outs[i], q_idx, "noalloc case %d" % i)


def test_noalloc_attention_repeat_is_deterministic():
    """Two calls with the same input give the same bytes (the scratch keeps the last call's
    partials, which the next call overwrites before reading)."""
    nv = _nv()
    q, k, v = _inputs(3, 300, 5000, 44)
    qd, kq, vq = q.to(dev()), nv.kv_quantize(k.to(dev())), nv.kv_quantize(v.to(dev()))
    a = nv.kv_attention_noalloc(qd, kq, vq, 4999)
    b = nv.kv_attention_noalloc(qd, kq, vq, 4999)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
