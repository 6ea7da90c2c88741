"""Seeded synthetic inputs shaped like a 5B video DiT's linears and KV cache.

This module only draws random tensors; it holds none of the NVFP4 arithmetic,
so the oracle side (tests) and the GPU side (binding, bench) can both use it.
The LongLive-2.0 pages (d9249.github.io review, "Evidence" section: the 5B
model at 1280x720; d9249 "Core idea": multi-shot attention sinks) give no
tensor shapes; the sizes below are hidden 3072, FFN 14336, 24 heads x 128,
65,536 cached tokens.

Recipes (every draw is torch.randn/rand in fp32 on the CPU from
torch.Generator seeded 1000*cfg + t, t = 0 activations/K, 1 weights/V,
2 auxiliary draws; bf16 tensors are the fp32 draws rounded to nearest even):
  1  A, B fp32 [256, 256] ~ N(0, 1)
  2  A bf16 [4096, 3072] ~ N(0, 1), entries with an i.i.d. Bernoulli(0.005)
     mask scaled x20 (outliers);  W bf16 [3072, 3072] ~ N(0, 0.02)
  3  A bf16 [16384, 3072] = std_k * N(0, 1), std_k = exp(0.5 z_k), z ~ N(0, 1)
     per input channel k;  W bf16 [14336, 3072] ~ N(0, 0.02)
  4  A bf16 [16384, 14336] = GELU(N(0, 1)) (erf form, fp32);
     W bf16 [3072, 14336] ~ N(0, 0.01)
  5  K, V bf16 [24, 65536, 128] ~ N(0, 1), tokens 0..3 of every head x8
     (attention-sink tokens); queries of a new chunk attending that cache
     bf16 [24, 4096, 128] ~ N(0, 1) (t = 2)
  backward of a linear (configs 2-4): the output gradient dY bf16 [M, N] =
     2^-12 * s_m * N(0, 1), s_m = exp(0.5 z_m) per token m (t = 3, z: t = 4);
     with A and W of the config it feeds dX = dY W and dW = dY^T A
  adaLN quantizer input (config 3 sizes): pre-norm hidden states x bf16
     [16384, 3072] = m_t + std_k * N(0, 1) (std_k as config 3, per-token mean
     m_t ~ N(0, 0.5^2), t = 5 / 6), modulation shift, scale fp32 [4, 3072]
     ~ N(0, 0.5^2) (t = 7), one per group of 4096 tokens
Sizes can be overridden (same recipe) for small parity cases.
"""
import torch

CONFIGS = {
    1: dict(workload="nvfp4_gemm_256_f32", M=256, N=256, K=256, a_dtype="f32", c_dtype="f32"),
    2: dict(workload="dit_attn_proj_4096x3072x3072", M=4096, N=3072, K=3072, a_dtype="bf16", c_dtype="bf16"),
    3: dict(workload="dit_ffn_up_fused_16384x14336x3072", M=16384, N=14336, K=3072, a_dtype="bf16",
            c_dtype="bf16"),
    4: dict(workload="dit_ffn_down_16384x3072x14336", M=16384, N=3072, K=14336, a_dtype="bf16",
            c_dtype="bf16"),
    5: dict(workload="nvfp4_kv_cache_24x65536x128", H=24, T=65536, D=128),
}


def generator(cfg, t):
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * cfg + t)
    return g


def activations(cfg, M=None, K=None):
    """Activation matrix A [M, K] of config cfg (CPU tensor)."""
    c = CONFIGS[cfg]
    M = c["M"] if M is None else M
    K = c["K"] if K is None else K
    if cfg == 1:
        return torch.randn(M, K, generator=generator(1, 0), dtype=torch.float32)
    a = torch.randn(M, K, generator=generator(cfg, 0), dtype=torch.float32)
    if cfg == 2:
        mask = torch.rand(M, K, generator=generator(2, 2), dtype=torch.float32) < 0.005
        a = torch.where(mask, a * 20.0, a)
    elif cfg == 3:
        z = torch.randn(K, generator=generator(3, 2), dtype=torch.float32)
        a = a * torch.exp(0.5 * z)[None, :]
    elif cfg == 4:
        a = torch.nn.functional.gelu(a, approximate="none")
    return a.to(torch.bfloat16)


def weights(cfg, N=None, K=None):
    """Weight matrix W [N, K] of config cfg (CPU tensor)."""
    c = CONFIGS[cfg]
    N = c["N"] if N is None else N
    K = c["K"] if K is None else K
    w = torch.randn(N, K, generator=generator(cfg, 1), dtype=torch.float32)
    if cfg == 1:
        return w
    std = {2: 0.02, 3: 0.02, 4: 0.01}[cfg]
    return (w * std).to(torch.bfloat16)


def output_grads(cfg, M=None, N=None):
    """Output gradient dY [M, N] of the linear of config cfg (CPU tensor, bf16)."""
    c = CONFIGS[cfg]
    M = c["M"] if M is None else M
    N = c["N"] if N is None else N
    g = torch.randn(M, N, generator=generator(cfg, 3), dtype=torch.float32)
    z = torch.randn(M, generator=generator(cfg, 4), dtype=torch.float32)
    return (g * (2.0 ** -12) * torch.exp(0.5 * z)[:, None]).to(torch.bfloat16)


def adaln_inputs(M=16384, K=3072, rows_per_group=4096):
    """(x bf16 [M, K], shift f32 [G, K], scale f32 [G, K], rows_per_group) of the fused adaLN quantizer."""
    x = torch.randn(M, K, generator=generator(3, 5), dtype=torch.float32)
    z = torch.randn(K, generator=generator(3, 2), dtype=torch.float32)
    m = torch.randn(M, 1, generator=generator(3, 6), dtype=torch.float32) * 0.5
    x = (x * torch.exp(0.5 * z)[None, :] + m).to(torch.bfloat16)
    G = (M + rows_per_group - 1) // rows_per_group
    mods = torch.randn(2, G, K, generator=generator(3, 7), dtype=torch.float32) * 0.5
    return x, mods[0].contiguous(), mods[1].contiguous(), rows_per_group


def kv_cache(H=None, T=None, D=None, sinks=4):
    """(K, V) bf16 [H, T, D] of the KV-cache workload (CPU tensors)."""
    c = CONFIGS[5]
    H = c["H"] if H is None else H
    T = c["T"] if T is None else T
    D = c["D"] if D is None else D
    out = []
    for t in (0, 1):
        x = torch.randn(H, T, D, generator=generator(5, t), dtype=torch.float32)
        x[:, :sinks, :] *= 8.0
        out.append(x.to(torch.bfloat16))
    return tuple(out)


def attention_queries(H=24, Tq=4096, D=128):
    """Queries of a new chunk attending the NVFP4 KV cache: bf16 [H, Tq, D] ~ N(0, 1), seed 1000 * 5 + 2."""
    return torch.randn(H, Tq, D, generator=generator(5, 2)).to(torch.bfloat16)


def bf16_bits(t):
    """uint16 numpy view of a bf16 CPU tensor (for the oracle)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
