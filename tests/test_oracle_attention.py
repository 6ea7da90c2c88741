"""Pins of the oracle's NVFP4-KV attention (orc_kv_attention) against things
other than itself: torch's fp64 scaled_dot_product_attention (a library
routine) on K/V decoded here from the format definition, and closed forms and
invariants of softmax attention."""
import numpy as np
import pytest
import torch

import oracle
import workloads

# E2M1 nibble values (bit 3 sign, bits 2:1 exponent with bias 1, bit 0 mantissa)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _e4m3(b):
    b = b.astype(np.int64)
    e, m = b >> 3, b & 7
    return np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))


def _decode(cache, T):
    """Exact fp64 rows of an NVFP4 cache (codes [H,Tc,D/2], scales [H,Tc,D/16], s_g [H]), first T tokens."""
    codes, scales, hs = cache
    codes, scales = codes[:, :T], scales[:, :T]
    vals = np.empty(codes.shape[:2] + (codes.shape[2] * 2,))
    vals[..., 0::2] = _E2M1[codes & 15]
    vals[..., 1::2] = _E2M1[codes >> 4]
    return vals * np.repeat(_e4m3(scales), 16, axis=2) * hs.astype(np.float64)[:, None, None]


def _bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _caches(H, T, D, seed):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn(H, T, D, generator=g) * 1.5).to(torch.bfloat16)
    v = torch.randn(H, T, D, generator=g).to(torch.bfloat16)
    return oracle.kv_quantize(workloads.bf16_bits(k)), oracle.kv_quantize(workloads.bf16_bits(v))


def _queries(H, Tq, D, seed, s=1.0):
    g = torch.Generator().manual_seed(seed)
    return workloads.bf16_bits((torch.randn(H, Tq, D, generator=g) * s).to(torch.bfloat16))


@pytest.mark.parametrize("H,Tq,Tc,T,D", [(2, 7, 64, 50, 32), (1, 3, 300, 300, 128), (3, 4, 97, 1, 16)])
def test_attention_matches_torch_sdpa_fp64(H, Tq, Tc, T, D):
    kc, vc = _caches(H, Tc, D, Tc + D)
    q = _queries(H, Tq, D, H + Tq, s=2.0)
    scale = 1.0 / np.sqrt(D)
    out, _ = oracle.kv_attention(q, kc, vc, T, scale)
    k, v = torch.from_numpy(_decode(kc, T)), torch.from_numpy(_decode(vc, T))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(_bf16_vals(q)), k, v, scale=scale)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12 * np.abs(ref.numpy()).max())


def test_attention_identical_keys_average_values():
    """All keys equal: every weight is 1, the output is the mean of the values."""
    H, T, D = 2, 33, 64
    g = torch.Generator().manual_seed(5)
    k = torch.randn(H, 1, D, generator=g).expand(H, T, D).contiguous().to(torch.bfloat16)
    v = torch.randn(H, T, D, generator=g).to(torch.bfloat16)
    kc, vc = oracle.kv_quantize(workloads.bf16_bits(k)), oracle.kv_quantize(workloads.bf16_bits(v))
    out, _ = oracle.kv_attention(_queries(H, 5, D, 9), kc, vc, T, 0.3)
    want = _decode(vc, T).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), rtol=1e-13, atol=1e-15)


def test_attention_single_token_returns_its_value():
    kc, vc = _caches(3, 20, 32, 1)
    out, wabs = oracle.kv_attention(_queries(3, 4, 32, 2), kc, vc, 1, 0.7)
    v0 = _decode(vc, 1)
    assert np.array_equal(out, np.broadcast_to(v0, out.shape))
    assert np.array_equal(wabs, np.abs(out))


def test_attention_ignores_rows_past_kv_tokens():
    kc, vc = _caches(2, 80, 32, 3)
    q = _queries(2, 6, 32, 4)
    a, _ = oracle.kv_attention(q, kc, vc, 50, 0.2)
    kc2 = (kc[0].copy(), kc[1].copy(), kc[2])
    vc2 = (vc[0].copy(), vc[1].copy(), vc[2])
    kc2[0][:, 50:] ^= 0x5A
    vc2[1][:, 50:] = 0x40
    b, _ = oracle.kv_attention(q, kc2, vc2, 50, 0.2)
    assert np.array_equal(a, b)


def test_attention_token_permutation_invariant():
    kc, vc = _caches(2, 64, 32, 6)
    q = _queries(2, 5, 32, 7, s=3.0)
    perm = np.random.default_rng(0).permutation(64)
    kp = (kc[0][:, perm], kc[1][:, perm], kc[2])
    vp = (vc[0][:, perm], vc[1][:, perm], vc[2])
    a, wa = oracle.kv_attention(q, kc, vc, 64, 0.25)
    b, wb = oracle.kv_attention(q, kp, vp, 64, 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(wa, wb, rtol=1e-12)


def test_attention_output_within_weighted_magnitude():
    kc, vc = _caches(2, 100, 64, 8)
    out, wabs = oracle.kv_attention(_queries(2, 9, 64, 9, s=4.0), kc, vc, 100, 0.125)
    assert (np.abs(out) <= wabs * (1 + 1e-12)).all()
    assert (wabs <= np.abs(_decode(vc, 100)).max(axis=1, keepdims=True) * (1 + 1e-12)).all()


@pytest.mark.parametrize("H,Tq,Tc,T,D", [(2, 5, 80, 70, 32), (1, 3, 300, 257, 128)])
def test_attention_normaliser_matches_logsumexp(H, Tq, Tc, T, D):
    """The normaliser sum_j exp(s_j - max s) equals exp(logsumexp(s) - max s) computed by torch
    (a library routine) from scores formed here out of the decoded rows; it is >= 1."""
    kc, vc = _caches(H, Tc, D, 3 * Tc + D)
    q = _queries(H, Tq, D, 7 * H + Tq, s=3.0)
    scale = 1.0 / np.sqrt(D)
    _, _, lsum = oracle.kv_attention(q, kc, vc, T, scale, return_norm=True)
    s = torch.einsum("hqd,htd->hqt", torch.from_numpy(_bf16_vals(q)), torch.from_numpy(_decode(kc, T))) * scale
    want = torch.exp(torch.logsumexp(s, dim=-1) - s.max(dim=-1).values).numpy()
    np.testing.assert_allclose(lsum, want, rtol=1e-12)
    assert (lsum >= 1.0).all()
    sub, _, lsub = oracle.kv_attention(q, kc, vc, T, scale, q_idx=np.array([2, 0]), return_norm=True)
    np.testing.assert_array_equal(lsub, lsum[:, [2, 0]])
