"""Shared helpers of the GPU parity tests: run the HIP library through its
binding and compare with the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import oracle
import workloads


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def oracle_input(x_cpu):
    """numpy view the oracle takes: float32 values or bf16 bit patterns."""
    if x_cpu.dtype == torch.float32:
        return x_cpu.contiguous().numpy()
    if x_cpu.dtype == torch.bfloat16:
        return workloads.bf16_bits(x_cpu)
    raise TypeError(x_cpu.dtype)


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def assert_quant_equal(gpu, orc, label=""):
    gc, gs, gg = gpu
    oc, os_, og = orc
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    gg = gg.cpu().numpy().reshape(-1)
    og = np.asarray(og, np.float32).reshape(-1)
    assert np.array_equal(f32_bits(gg), f32_bits(og)), "%s: s_g %r vs oracle %r" % (label, gg, og)
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, "%s: %d scale bytes differ, first at %s: %d vs %d" % (
        label, len(bad_s), bad_s[0], gs[tuple(bad_s[0])], os_[tuple(bad_s[0])])
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, "%s: %d code bytes differ, first at %s: %#x vs %#x" % (
        label, len(bad_c), bad_c[0], gc[tuple(bad_c[0])], oc[tuple(bad_c[0])])


def bf16_to_f64(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def half_ulp_bf16(c):
    """Half a bf16 ulp at |c| (c exactly a bf16 value), 0 for c = 0."""
    a = np.abs(c)
    _, e = np.frexp(a)  # a = f * 2^e, f in [0.5, 1)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.where(a > 0, 0.5 * ulp, 0.5 * np.ldexp(1.0, -133))


def check_gemm_bound(c_out, ref, tot, bf16_out, label=""):
    """max |C - ref| <= 1e-5 * sum|a b| (+ half a bf16 ulp of C for bf16 output)."""
    c = np.asarray(c_out, np.float64)
    err = np.abs(c - ref)
    bound = 1e-5 * tot + (half_ulp_bf16(c) if bf16_out else 0.0)
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err > 0, np.inf, 0))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, "%s: error exceeds bound (worst err/bound %.3g at %s)" % (
        label, worst, np.unravel_index(int(ratio.argmax()), ratio.shape))
    return worst


def c_to_f64(c_dev):
    if c_dev.dtype == torch.bfloat16:
        return bf16_to_f64(c_dev.cpu().view(torch.int16).numpy().view(np.uint16))
    return c_dev.cpu().numpy().astype(np.float64)


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
E4M3 = np.array([oracle.e4m3_value(b) for b in range(127)], np.float64)


def _unpack_codes(codes):
    lo, hi = codes & 0xF, codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def check_quant_near_exact(codes, scales, y, tau, s_g, label):
    """GPU codes / scales (device tensors) of values the kernel computed in fp32, against the
    oracle's exact quantization of the fp64 values y with the same s_g: a scale byte or code may
    differ only where the exact block maximum or element lies within tau (per element) of the
    boundary between the two neighbouring values, and such elements must be rare."""
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    oc, os_, _ = oracle.quantize(y, np.float32(s_g))
    rows, k = y.shape
    sg = float(np.float32(s_g))
    amax_b = np.abs(y).reshape(rows, k // 16, 16).max(axis=2)
    tau_b = tau.reshape(rows, k // 16, 16).max(axis=2)
    bad_b = np.argwhere(gs != os_)
    for r, b in bad_b:
        lo, hi = sorted((int(gs[r, b]), int(os_[r, b])))
        assert hi == lo + 1, "%s: block (%d,%d) scale bytes %d / %d not adjacent" % (label, r, b, gs[r, b], os_[r, b])
        mid = 0.5 * (E4M3[lo] + E4M3[hi]) * 6 * sg
        assert abs(amax_b[r, b] - mid) <= tau_b[r, b], "%s: block (%d,%d) scale differs away from a boundary" % (
            label, r, b)
    same_block = np.repeat(gs == os_, 16, axis=1)
    gq, oq = _unpack_codes(gc), _unpack_codes(oc)
    diff = np.argwhere((gq != oq) & same_block)
    S = np.repeat(E4M3[os_.astype(int)] * sg, 16, axis=1)
    for r, d in diff:
        m1, m2 = int(gq[r, d]) & 7, int(oq[r, d]) & 7
        v = abs(y[r, d])
        if m1 == m2:  # sign only: a value within tau of zero that rounds to magnitude 0
            assert m1 == 0 and v <= tau[r, d], "%s: (%d,%d) sign differs" % (label, r, d)
            continue
        lo, hi = sorted((m1, m2))
        same_sign = (int(gq[r, d]) >> 3) == (int(oq[r, d]) >> 3)
        assert hi == lo + 1 and (same_sign or lo == 0), "%s: (%d,%d) codes %#x / %#x not neighbours" % (
            label, r, d, gq[r, d], oq[r, d])
        mid = 0.5 * (E2M1[lo] + E2M1[hi]) * S[r, d]
        assert abs(v - mid) <= tau[r, d], "%s: (%d,%d) code %#x vs %#x away from a boundary (|y| %.9g, mid %.9g)" % (
            label, r, d, gq[r, d], oq[r, d], v, mid)
    n_diff = len(diff) + 16 * len(bad_b)
    log(label, "elements off the exact rounding: %d of %d (%d blocks)" % (len(diff), y.size, len(bad_b)))
    assert n_diff <= 1e-4 * y.size + 16


def window_sample(n, window=64, seed=0):
    """One index in every `window`-wide window of 0 .. n-1 (the last one ragged), at offsets
    that run through every residue mod 32, plus 0 and n - 1.  Any output tile of the GEMM that is
    at least 2 windows wide therefore holds at least two sampled indices."""
    idx = [0, n - 1]
    for i, w0 in enumerate(range(0, n, window)):
        width = min(window, n - w0)
        idx.append(w0 + (17 * i + 5 + seed) % width)
    return np.unique(np.asarray(idx, np.int64))


def check_gemm_tiles(c, ao, bo, bf16_out, label, seed=0, tile=256):
    """GEMM output c (float64 [M, N]) against the oracle on the cross product of sampled rows and
    columns (window_sample of both) plus whole rows 0, M-1 and columns 0, N-1; asserts that every
    tile x tile output tile has at least 4 compared elements.  Returns the worst err / bound."""
    M, N = c.shape
    rows, cols = window_sample(M, seed=seed), window_sample(N, seed=seed + 3)
    cover = np.zeros(((M + tile - 1) // tile, (N + tile - 1) // tile), np.int64)
    np.add.at(cover, (rows[:, None] // tile, cols[None, :] // tile), 1)
    assert cover.min() >= 4, "%s: a %dx%d tile has only %d sampled outputs" % (label, tile, tile, cover.min())
    ref, tot = oracle.gemm_ref(*ao, *bo, rows=rows, cols=cols)
    w = check_gemm_bound(c[np.ix_(rows, cols)], ref, tot, bf16_out, label + " tiles")
    edge_r, edge_c = np.array([0, M - 1]), np.array([0, N - 1])
    ref, tot = oracle.gemm_ref(*ao, *bo, rows=edge_r)
    w = max(w, check_gemm_bound(c[edge_r], ref, tot, bf16_out, label + " rows"))
    ref, tot = oracle.gemm_ref(*ao, *bo, cols=edge_c)
    w = max(w, check_gemm_bound(c[:, edge_c], ref, tot, bf16_out, label + " cols"))
    log(label, "compared %d x %d sampled outputs (every %dx%d tile >= %d) + edges, worst err/bound %.3g" % (
        rows.size, cols.size, tile, tile, cover.min(), w))
    return w
