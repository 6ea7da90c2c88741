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
