"""GPU parity of kv_attention (softmax attention over a packed NVFP4 KV cache)
with the oracle's fp64 attention over the same caches.

Tolerance per output element o[h][i][d] (ref, wabs, L from the oracle):
  |o - ref| <= half_ulp_bf16(ref) + 2^-9 * wabs + 2^-25 * T * vmax[h][d] / (L (1 - 2^-6))
where wabs = sum_j w_j |v_jd| / sum_j w_j, L = sum_j w_j (w_j = exp(s_j - max s),
so L >= 1), T the attended tokens and vmax the largest |v_jd|.  The kernel's
operands are exact (bf16 queries, K and V decoded exactly), so its error comes
from: the probabilities rounded to fp16 for the second product (2^-11 relative,
or 2^-25 absolute below 2^-14: at most T 2^-25 vmax in the un-normalised sum,
which the kernel divides by its own normaliser l), the fp32 sums of scores and
of the output (about 2^-11 of wabs together at these sizes), the fp32 exp2 (all
within 2^-9 wabs), and the final bf16 rounding (half an ulp of ref).  The
kernel's l differs from L by those same roundings, at most 2^-9 + 2^-11 of L
plus T 2^-25 <= 2^-9 absolute (its running maximum is the largest computed
score, so its largest weight is 1), hence l >= L (1 - 2^-6).  The bound must
stay below |ref| for at least 90% of the compared elements (checked), so that
it cannot pass a wrong output wholesale."""
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


def _run(H, Tq, Tc, T, seed, qscale=1.0, scale=None, q_idx=None, workspaces=(None,)):
    """workspaces: kv_attention's workspace per run (None: the preferred split;
    an int: a workspace of that many bytes, 0 turning the split off)."""
    nv = _nv()
    D = 128
    k, v = workloads.kv_cache(H, Tc, D, sinks=min(4, Tc))
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(H, Tq, D, generator=g) * qscale).to(torch.bfloat16)
    scale = D ** -0.5 if scale is None else scale
    kq, vq = nv.kv_quantize(k.to(dev())), nv.kv_quantize(v.to(dev()))
    outs = []
    for w in workspaces:
        wt = None if w is None else torch.empty(w, dtype=torch.uint8, device=dev())
        outs.append(nv.kv_attention(q.to(dev()), kq, vq, T, scale, workspace=wt))
    torch.cuda.synchronize()
    ok, ov = oracle.kv_quantize(workloads.bf16_bits(k)), oracle.kv_quantize(workloads.bf16_bits(v))
    for g_, o_ in zip(list(kq) + list(vq), list(ok) + list(ov)):  # the caches fed to the oracle are its own
        assert np.array_equal(g_.cpu().numpy().view(np.uint8), np.asarray(o_).view(np.uint8))
    ref, wabs, lsum = oracle.kv_attention(workloads.bf16_bits(q), ok, ov, T, scale, q_idx=q_idx, return_norm=True)
    vf = np.stack([oracle.dequantize(ov[0][h, :T], ov[1][h, :T], ov[2][h], "f32") for h in range(H)])
    vmax = np.abs(vf).max(axis=1)[:, None, :]
    sub = 2.0 ** -25 * T * vmax / (lsum[..., None] * (1.0 - 2.0 ** -6))
    live = float((half_ulp_bf16(ref) + 2.0 ** -9 * wabs + sub < np.abs(ref)).mean())
    assert live >= 0.9, "the bound exceeds |ref| on %.1f%% of the elements" % (100 * (1 - live))
    for w, o in zip(workspaces, outs):
        got = c_to_f64(o)
        if q_idx is not None:
            got = got[:, q_idx]
        err = np.abs(got - ref)
        tol = np.maximum(half_ulp_bf16(ref), half_ulp_bf16(got)) + 2.0 ** -9 * wabs + sub
        ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err > 0, np.inf, 0.0))
        worst = float(ratio.max())
        log("attention", H, Tq, Tc, T, "workspace", w, "worst err/tol %.3g, max err %.3g, bound < |ref| on %.1f%%" % (
            worst, err.max(), 100 * live))
        assert worst <= 1.0, "workspace %s: error exceeds the bound: worst err/tol %.3g at %s" % (
            w, worst, np.unravel_index(int(ratio.argmax()), err.shape))


@pytest.mark.parametrize("H,Tq,Tc,T", [(2, 100, 200, 150), (1, 1, 64, 1), (3, 300, 4096, 4096), (2, 257, 1000, 999),
                                       (1, 512, 130, 65)])
def test_attention_small(H, Tq, Tc, T):
    _run(H, Tq, Tc, T, seed=H * 7 + Tq)


def test_attention_peaked_softmax():
    """Large queries: sharply peaked weights, the running max changes often."""
    _run(2, 300, 2048, 2000, seed=3, qscale=6.0)


def test_attention_negative_and_zero_scale():
    """A negative softmax factor (folded into the queries' signs by the kernel)
    and a zero one (every weight equal: the plain mean of the values)."""
    _run(2, 100, 300, 250, seed=5, scale=-0.2)
    _run(1, 64, 200, 200, seed=6, scale=0.0)


def test_attention_full_cache_sampled_queries():
    """The 24-head 65,536-token cache, 1,024 queries per head; sampled query rows."""
    _run(24, 1024, 65536, 65536, seed=11, q_idx=np.array([0, 1, 255, 256, 511, 777, 1023]))


def test_attention_split_cache_modes():
    """The split-cache path against the same oracle: the preferred split (20
    ranges of 4 blocks, the last one ragged, for 6 workgroups over 79 cache
    blocks), a workspace that fits two ranges, and none (one pass)."""
    H, Tq = 3, 300
    per_range = H * Tq * 520
    assert _nv().kv_attention_workspace_size(H, Tq, 4999) > 2 * per_range
    _run(H, Tq, 5000, 4999, seed=21, workspaces=(None, 2 * per_range + 100, 0))


def test_attention_split_one_query():
    """One query per head over a long cache: most workgroups hold one range of
    a single query's cache."""
    _run(4, 1, 20000, 19990, seed=22, qscale=3.0, workspaces=(None, 0))
