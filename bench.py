#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

One step is the DiT FFN up-projection of a long-video chunk as a W4A4 NVFP4
linear: the bf16 activations A [16384, 3072] are quantized to NVFP4 (amax,
per-tensor scale, per-16 E4M3 scales and E2M1 codes) and multiplied with the
pre-quantized weights W [14336, 3072] (C = A . W^T, bf16 out).  The step is
the same kernel sequence nvfp4_gemm_fused_act enqueues, issued as
nvfp4_quantize + nvfp4_gemm so that HIP events can bracket the GEMM kernel.
Weights are quantized once, outside the timed region.  Inputs are seeded
synthetic tensors (workloads/), resident in HBM before timing starts.

Printed: one JSON line with the step throughput (TFLOP/s = 2 M N K / step
time), the GEMM kernel's roofline against the fp16/bf16 dense MFMA peak,
secondary HBM throughputs (activation quantize of the FFN down-projection
input, NVFP4 KV-cache round trip), and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps 30] [--warmup 10]

Before the W warm-up steps the step runs for SETTLE_S seconds: the GPU's
clocks take tens of milliseconds of sustained load to settle (the GEMM's
kernel time drifts by up to 30% over its first ~30 launches), and the timed
steps are meant to measure the steady state.

roofline.traffic is the GEMM kernel's HBM bytes per launch from rocprofv3
FETCH_SIZE / WRITE_SIZE counters (profiles/), scaled by what the same
counters read for a 1 GiB device copy; it is reported only while the GEMM
sources hash to the ones the counters were taken on, else null.
"""
import argparse
import hashlib
import json
import os
import sys
import time

METRIC = "W4A4 NVFP4 GEMM TFLOP/s (M16384 K3072 N14336) + quant/dequant HBM GB/s"
MFMA_PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
SETTLE_S = 0.5
GEMM_KERNEL = "gemm_w4a4_fast_kernel"
GEMM_SOURCES = ("long_video_dit_amd/csrc/nvfp4_gemm.hip", "long_video_dit_amd/csrc/nvfp4_device.h")
# HBM byte counters of one GEMM launch (FFN up-projection, bf16 out), KiB per dispatch, and the
# factors that map them to bytes (a 1 GiB copy reads FETCH_SIZE = 512 MiB, WRITE_SIZE = 1 GiB).
# Taken with profiles/gemm_w4a4_fast_kernel_ffn_up_16384x14336x3072.md's commands.
GEMM_COUNTERS = {"sources_sha256": "fa4ee1ae5d532974c8c12ff00a60349cc5df1e0f45c307c224bf6b88d6c674f8",
                 "fetch_kib": 281189.50, "write_kib": 458783.45, "fetch_scale": 2.0, "write_scale": 1.0}
# Whole-pass HBM bytes per element (bf16 data, 4-bit code + one 8-bit scale per 16 elements).
B_AMAX = 2.0
B_ENCODE = 2.0 + 0.5 + 1.0 / 16
B_ADALN = 2.0 + B_ENCODE  # fused adaLN quantizer: x read twice (amax pass, encode pass), codes + scales written
B_DEQUANT = 0.5 + 1.0 / 16 + 2.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--no-secondary", action="store_true", help="skip the quantize / KV-cache bandwidth lines")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--all-configs", action="store_true",
                   help="instead of the step: time every workload (quantize, GEMM, KV cache) and the oracle "
                        "on a bounded sample of each, one JSON line")
    return p.parse_args()


def events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


FLUSH_BYTES = 1 << 30  # written between cold calls: four times the 256 MB Infinity Cache (MALL)


def time_cold(torch, fn, flush, steps):
    """Average ms of fn() with the caches cold: before each call a 1 GiB buffer is
    written (evicting L2 and MALL), outside the HIP-event window of the call."""
    pairs = [events(torch, 2) for _ in range(steps)]
    for s, e in pairs:
        flush.fill_(1.0)
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in pairs) / steps


def time_calls(torch, fn, steps, warmup):
    """Average ms of fn() over `steps` calls, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = events(torch, 2)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def time_calls_dist(torch, fn, steps, warmup):
    """Per-call ms of fn() over `steps` calls, an HIP event pair around each
    call on the current stream: (mean, p10, median, p90).  Each pair adds the
    call's launch latency, a few us, so the reported means come from
    time_calls (one pair around back-to-back calls) and these give the spread."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    pairs = [events(torch, 2) for _ in range(steps)]
    for s, e in pairs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return dist([s.elapsed_time(e) for s, e in pairs])


def dist(ms):
    """(mean, p10, median, p90) of a list of times, rounded to 0.1 us."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return tuple(round(float(v), 4) for v in (a.mean(), *np.percentile(a, [10, 50, 90])))


def flop_of(M, N, K):
    return 2.0 * M * N * K


def time_graph(torch, fn, calls=20, replays=5):
    """Average ms of fn() with `calls` calls captured in one HIP graph and the
    graph replayed `replays` times (HIP events around the replays): the GPU
    time of a call without the binding's per-call host time, which exceeds
    the kernel time of the shortest calls.  fn must write preallocated buffers
    only."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    s, e = events(torch, 2)
    s.record()
    for _ in range(replays):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / (replays * calls)
    del graph
    return ms


def sources_sha256(root):
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm_traffic(root):
    """HBM bytes per GEMM launch from the recorded counters, or None when the
    kernel sources changed since they were taken."""
    c = GEMM_COUNTERS
    if c["sources_sha256"] is None or c["sources_sha256"] != sources_sha256(root):
        return None
    return int(round((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the NVFP4 hot path runs on a single MI355X here; "
              "--gpus %d is not supported (multi-GPU sharding is a design note only)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import workloads
    from long_video_dit_amd import nvfp4

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.all_configs:
        print(json.dumps({"all_configs": all_configs(torch, nvfp4, workloads, dev, args.steps, args.warmup)}),
              flush=True)
        return
    cfg = workloads.CONFIGS[3]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    flop = 2.0 * M * N * K

    log("generating inputs", M, N, K)
    a = workloads.activations(3).to(dev)
    w = workloads.weights(3).to(dev)
    wq = nvfp4.quantize(w)  # weights: once, outside the timed region
    del w
    aq = (torch.empty(M, K // 2, dtype=torch.uint8, device=dev),
          torch.empty(M, K // 16, dtype=torch.uint8, device=dev),
          torch.empty(1, dtype=torch.float32, device=dev))
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    gemm_s, gemm_e = events(torch, args.steps), events(torch, args.steps)

    def step(i=None):
        nvfp4.quantize(a, out=aq[:2], s_g_out=aq[2])
        if i is not None:
            gemm_s[i].record()
        nvfp4.gemm(aq, wq, out=c)
        if i is not None:
            gemm_e[i].record()

    log("settling clocks for %.1f s" % SETTLE_S)
    settle(torch, step)
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing", args.steps, "steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gemm_times = [s.elapsed_time(e) for s, e in zip(gemm_s, gemm_e)]
    gemm_ms = sum(gemm_times) / args.steps
    _, gemm_p10, gemm_p50, gemm_p90 = dist(gemm_times)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (gemm_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "M": M, "N": N, "K": K, "a_dtype": "bf16", "c_dtype": "bf16",
                   "w_format": "nvfp4", "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": GEMM_KERNEL, "achieved": round(achieved, 1),
                     "peak": MFMA_PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_F16_TFLOPS, 4), "traffic": gemm_traffic(root),
                     "algorithmic_bytes": M * (K // 2 + K // 16) + N * (K // 2 + K // 16) + 2 * M * N + 8,
                     "gemm_ms": round(gemm_ms, 4), "gemm_ms_p10_p50_p90": [gemm_p10, gemm_p50, gemm_p90]},
    }
    log("step %.3f ms, gemm %.3f ms -> %.1f TFLOP/s step, %.1f TFLOP/s gemm" % (ms_per_step, gemm_ms, value,
                                                                             achieved))

    if not args.no_secondary:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        cold_ms = time_cold(torch, step, flush, args.steps)
        quant = lambda: nvfp4.quantize(a, out=aq[:2], s_g_out=aq[2])
        cold_q = time_cold(torch, quant, flush, 10)
        warm_q = time_calls(torch, quant, 10, 2)
        del flush
        out["secondary"] = secondary(torch, nvfp4, workloads, dev, a, aq)
        qb = M * K * (B_AMAX + B_ENCODE)
        out["secondary"]["cold"] = {
            "note": "a 1 GiB buffer written before every call, outside the event window (the MALL is 256 MB)",
            "step_ffn_up": {"ms": round(cold_ms, 4), "TFLOP/s": round(flop / (cold_ms * 1e-3) / 1e12, 1),
                            "warm_ms": round(ms_per_step, 4)},
            "quantize_ffn_up_act": {"shape": [M, K], "ms": round(cold_q, 4),
                                    "GB/s": round(qb / (cold_q * 1e-3) / 1e9, 1), "warm_ms": round(warm_q, 4),
                                    "warm_GB/s": round(qb / (warm_q * 1e-3) / 1e9, 1)},
            **out["secondary"].pop("_cold")}
    if args.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 2 * x.numel() * 4
    del c
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(workloads, M, N, K)
    print(json.dumps(out), flush=True)


def secondary(torch, nvfp4, workloads, dev, a3, aq3):
    """HBM throughput of the quantizer and the NVFP4 KV-cache round trip, the attention over
    the packed cache, the backward operands and GEMMs of the FFN up-projection, and the
    adaLN-fused quantizer."""
    res = {}
    # activation quantize of the FFN down-projection input (bf16 [16384, 14336], 470 MB)
    a4 = workloads.activations(4).to(dev)
    M4, K4 = a4.shape
    q4 = (torch.empty(M4, K4 // 2, dtype=torch.uint8, device=dev),
          torch.empty(M4, K4 // 16, dtype=torch.uint8, device=dev),
          torch.empty(1, dtype=torch.float32, device=dev))
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    cold = {}
    q4f = lambda: nvfp4.quantize(a4, out=q4[:2], s_g_out=q4[2])
    settle(torch, q4f, 0.3)
    ms_c = time_cold(torch, q4f, flush, 10)
    ms = time_calls(torch, q4f, 30, 2)
    n = a4.numel()
    cold["quantize_ffn_down_act"] = {"shape": [M4, K4], "ms": round(ms_c, 4),
                                     "GB/s": round(n * (B_AMAX + B_ENCODE) / (ms_c * 1e-3) / 1e9, 1)}
    res["quantize_ffn_down_act"] = {"shape": [M4, K4], "ms": round(ms, 4),
                                    "GB/s": round(n * (B_AMAX + B_ENCODE) / (ms * 1e-3) / 1e9, 1),
                                    "bytes_per_elem": B_AMAX + B_ENCODE}
    # the same with FourOverSix block scaling (two candidate scales per block)
    ms = time_calls(torch, lambda: nvfp4.quantize(a4, out=q4[:2], s_g_out=q4[2], four_over_six=True), 10, 2)
    res["quantize_ffn_down_act_four_over_six"] = {"shape": [M4, K4], "ms": round(ms, 4),
                                                  "GB/s": round(n * (B_AMAX + B_ENCODE) / (ms * 1e-3) / 1e9, 1),
                                                  "bytes_per_elem": B_AMAX + B_ENCODE}
    del a4, q4
    # NVFP4 KV cache: K and V bf16 [24, 65536, 128], quantize + dequantize
    k, v = workloads.kv_cache()
    k, v = k.to(dev), v.to(dev)
    H, T, D = k.shape
    qk, qv = nvfp4.kv_quantize(k), nvfp4.kv_quantize(v)
    ok, ov = torch.empty_like(k), torch.empty_like(v)

    def rt():
        nvfp4.kv_quantize(k, out=qk)
        nvfp4.kv_quantize(v, out=qv)
        nvfp4.kv_dequantize(*qk, out=ok)
        nvfp4.kv_dequantize(*qv, out=ov)

    settle(torch, rt, 0.3)
    ms = time_calls(torch, rt, 30, 2)
    ms_c = time_cold(torch, rt, flush, 10)
    n = 2 * k.numel()
    res["kv_cache_roundtrip"] = {"shape": [H, T, D], "tensors": 2, "ms": round(ms, 4),
                                 "GB/s": round(n * (B_AMAX + B_ENCODE + B_DEQUANT) / (ms * 1e-3) / 1e9, 1),
                                 "bytes": n * (B_AMAX + B_ENCODE + B_DEQUANT)}
    cold["kv_cache_roundtrip"] = {"ms": round(ms_c, 4),
                                  "GB/s": round(n * (B_AMAX + B_ENCODE + B_DEQUANT) / (ms_c * 1e-3) / 1e9, 1)}
    ms_qc = time_cold(torch, lambda: nvfp4.kv_quantize(k, out=qk), flush, 10)
    ms_dc = time_cold(torch, lambda: nvfp4.kv_dequantize(*qk, out=ok), flush, 10)
    cold["kv_quantize"] = {"ms": round(ms_qc, 4),
                           "GB/s": round(k.numel() * (B_AMAX + B_ENCODE) / (ms_qc * 1e-3) / 1e9, 1)}
    cold["kv_dequantize"] = {"ms": round(ms_dc, 4), "GB/s": round(k.numel() * B_DEQUANT / (ms_dc * 1e-3) / 1e9, 1)}
    del flush
    res["_cold"] = cold
    # attention of 4,096 new queries per head over the whole packed cache (K and V quantized above)
    Tq = 4096
    qa = workloads.attention_queries(H, Tq, D).to(dev)
    oa = torch.empty_like(qa)
    wsa = torch.empty(nvfp4.kv_attention_workspace_size(H, Tq, T, D), dtype=torch.uint8, device=dev)
    attn = lambda: nvfp4.kv_attention(qa, qk, qv, out=oa, workspace=wsa)
    settle(torch, attn)
    ms_a = time_calls(torch, attn, 10, 2)
    flop_a = 4.0 * H * Tq * T * D
    res["kv_attention"] = {"heads": H, "q_tokens": Tq, "kv_tokens": T, "head_dim": D, "ms": round(ms_a, 4),
                           "workspace_bytes": wsa.numel(),
                           "TFLOP/s": round(flop_a / (ms_a * 1e-3) / 1e12, 1),
                           "frac_of_fp16_peak": round(flop_a / (ms_a * 1e-3) / 1e12 / MFMA_PEAK_F16_TFLOPS, 4)}
    # RoPE fused into the append: the chunk's 4096 new keys per head rotated into the cache tail
    kn = qa.clone()
    ra = lambda: nvfp4.kv_rope_quantize_append(kn, qk, T - Tq)
    settle(torch, ra, 0.2)
    ms_r = time_calls(torch, ra, 10, 2)
    ms_rg = time_graph(torch, ra)
    res["kv_rope_append"] = {"heads": H, "tokens_new": Tq, "head_dim": D, "ms": round(ms_rg, 4),
                             "GB/s": round(kn.numel() * (2 + 0.5625) / (ms_rg * 1e-3) / 1e9, 1),
                             "timing": "HIP graph of 20 calls", "ms_eager": round(ms_r, 4)}
    del qa, oa, wsa, kn
    ms_q = time_calls(torch, lambda: nvfp4.kv_quantize(k, out=qk), 30, 2)
    ms_d = time_calls(torch, lambda: nvfp4.kv_dequantize(*qk, out=ok), 30, 2)
    ms_q46 = time_calls(torch, lambda: nvfp4.kv_quantize(k, out=qk, four_over_six=True), 10, 2)
    res["kv_quantize"] = {"ms": round(ms_q, 4), "GB/s": round(k.numel() * (B_AMAX + B_ENCODE) / (ms_q * 1e-3) / 1e9, 1)}
    res["kv_quantize_four_over_six"] = {
        "ms": round(ms_q46, 4), "GB/s": round(k.numel() * (B_AMAX + B_ENCODE) / (ms_q46 * 1e-3) / 1e9, 1)}
    res["kv_dequantize"] = {"ms": round(ms_d, 4), "GB/s": round(k.numel() * B_DEQUANT / (ms_d * 1e-3) / 1e9, 1)}
    # backward of the FFN up-projection: dY [16384, 14336] quantized along its rows (the wgrad
    # operand), dX = dY W (contracting 14336) and dW = dY^T A (contracting 16384)
    del k, v, qk, qv, ok, ov
    w3, dy = workloads.weights(3).to(dev), workloads.output_grads(3).to(dev)
    dyq, wtq, dytq, atq = nvfp4.quantize(dy), nvfp4.quantize_transposed(w3), nvfp4.quantize_transposed(dy), \
        nvfp4.quantize_transposed(a3)
    qt = lambda: nvfp4.quantize_transposed(dy, out=dytq[:2], s_g_out=dytq[2])
    settle(torch, qt)
    ms_t = time_calls(torch, qt, 10, 2)
    dx = torch.empty(dy.shape[0], w3.shape[1], dtype=torch.bfloat16, device=dev)
    dw = torch.empty(w3.shape, dtype=torch.bfloat16, device=dev)
    dgrad = lambda: nvfp4.gemm(dyq, wtq, out=dx)
    wgrad = lambda: nvfp4.gemm(dytq, atq, out=dw)
    settle(torch, dgrad)
    ms_dx = time_calls(torch, dgrad, 10, 2)
    ms_dw = time_calls(torch, wgrad, 10, 2)
    M3, N3, K3 = dy.shape[0], dy.shape[1], w3.shape[1]
    fl = 2.0 * M3 * N3 * K3
    res["backward_ffn_up"] = {
        "quantize_transposed_dY": {"shape": [M3, N3], "ms": round(ms_t, 4),
                                   "GB/s": round(dy.numel() * (B_AMAX + B_ENCODE) / (ms_t * 1e-3) / 1e9, 1)},
        "dgrad_dX_16384x3072x14336": {"ms": round(ms_dx, 4), "TFLOP/s": round(fl / (ms_dx * 1e-3) / 1e12, 1)},
        "wgrad_dW_14336x3072x16384": {"ms": round(ms_dw, 4), "TFLOP/s": round(fl / (ms_dw * 1e-3) / 1e12, 1)}}
    del w3, dy, dyq, wtq, dytq, atq, dx, dw
    # adaLN fused into the quantizer: pre-norm hidden states [16384, 3072], 4 modulation groups
    xa, sha, sca, rpg = workloads.adaln_inputs()
    xa, sha, sca = xa.to(dev), sha.to(dev), sca.to(dev)
    qa_ = nvfp4.adaln_quantize(xa, sha, sca, rpg)
    ada = lambda: nvfp4.adaln_quantize(xa, sha, sca, rpg, out=qa_[:2], s_g_out=qa_[2])
    settle(torch, ada)
    ms_ad = time_calls(torch, ada, 10, 2)
    res["adaln_quantize"] = {"shape": list(xa.shape), "groups": sha.shape[0], "ms": round(ms_ad, 4),
                             "GB/s": round(xa.numel() * B_ADALN / (ms_ad * 1e-3) / 1e9, 1),
                             "bytes_per_elem": B_ADALN}
    del xa, sha, sca, qa_
    res["hbm_peak_GB/s"] = HBM_PEAK_GBS
    log("secondary", json.dumps(res))
    return res


def all_configs(torch, nvfp4, workloads, dev, steps, warmup):
    """Every workload at full size: GPU times from HIP events (warm, after the
    clock-settling phase), and the CPU oracle timed on a bounded row sample
    and scaled linearly to the full size (quantize includes the full amax)."""
    import numpy as np
    import oracle

    res = {}
    for cfg in (1, 2, 3, 4):
        c = workloads.CONFIGS[cfg]
        a_cpu, w_cpu = workloads.activations(cfg), workloads.weights(cfg)
        a, w = a_cpu.to(dev), w_cpu.to(dev)
        M, K = a.shape
        N = w.shape[0]
        wq = nvfp4.quantize(w)
        aq = (torch.empty(M, K // 2, dtype=torch.uint8, device=dev),
              torch.empty(M, K // 16, dtype=torch.uint8, device=dev),
              torch.empty(1, dtype=torch.float32, device=dev))
        out = torch.float32 if c["c_dtype"] == "f32" else torch.bfloat16
        cbuf = torch.empty(M, N, dtype=out, device=dev)
        quant = lambda: nvfp4.quantize(a, out=aq[:2], s_g_out=aq[2])
        gemm = lambda: nvfp4.gemm(aq, wq, out=cbuf)
        quant()
        settle(torch, gemm)
        q_ms = time_calls(torch, quant, steps, warmup)
        g_ms = time_calls(torch, gemm, steps, warmup)
        _, *q_pct = time_calls_dist(torch, quant, steps, 0)
        _, *g_pct = time_calls_dist(torch, gemm, steps, 0)
        f_ms = time_calls(torch, lambda: nvfp4.gemm_fused_act(a, wq, out=cbuf, a_q=aq), steps, warmup)
        q_ms_g = time_graph(torch, quant)
        g_ms_g = time_graph(torch, gemm, calls=10 if flop_of(M, N, K) > 1e11 else 20)
        esz = a.element_size()
        qbytes = M * K * (2 * esz + 0.5625)
        flop = 2.0 * M * N * K
        # oracle on a bounded sample
        to_np = (lambda t: t.numpy()) if a_cpu.dtype == torch.float32 else workloads.bf16_bits
        an, wn = to_np(a_cpu), to_np(w_cpu)
        wo = oracle.quantize(wn)
        rows = min(M, max(1, int(2.0e9 / (2.0 * N * K))))  # about 2 s of fp64 dot products
        t0 = time.perf_counter()
        g = oracle.global_scale(oracle.amax(an))  # full tensor
        ta = time.perf_counter()
        ao = oracle.quantize(np.ascontiguousarray(an[:rows]), s_g=g)
        t1 = time.perf_counter()
        oracle.gemm_ref(*ao, *wo)
        t2 = time.perf_counter()
        oq_ms = (ta - t0) * 1e3 + (t1 - ta) * 1e3 * M / rows
        og_ms = (t2 - t1) * 1e3 * M / rows
        res[c["workload"]] = {
            "M": M, "N": N, "K": K, "a_dtype": c["a_dtype"], "c_dtype": c["c_dtype"],
            "quantize_ms": round(q_ms, 4), "quantize_GB/s": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
            "quantize_ms_p10_p50_p90": q_pct,
            "gemm_ms": round(g_ms, 4), "gemm_TFLOP/s": round(flop / (g_ms * 1e-3) / 1e12, 1),
            "gemm_ms_p10_p50_p90": g_pct,
            "gemm_frac_of_fp16_peak": round(flop / (g_ms * 1e-3) / 1e12 / MFMA_PEAK_F16_TFLOPS, 4),
            "fused_act_ms": round(f_ms, 4), "fused_act_TFLOP/s": round(flop / (f_ms * 1e-3) / 1e12, 1),
            "graph": {"note": "calls replayed from a HIP graph (no per-call host time)",
                      "quantize_ms": round(q_ms_g, 4), "quantize_GB/s": round(qbytes / (q_ms_g * 1e-3) / 1e9, 1),
                      "gemm_ms": round(g_ms_g, 4), "gemm_TFLOP/s": round(flop / (g_ms_g * 1e-3) / 1e12, 1)},
            "oracle_quantize_ms_est": round(oq_ms, 1), "oracle_gemm_ms_est": round(og_ms, 1),
            "oracle_sample_rows": rows, "oracle_threads": oracle.num_threads()}
        log("config", cfg, json.dumps(res[c["workload"]]))
        del a, w, wq, aq, cbuf
        torch.cuda.empty_cache()
    c = workloads.CONFIGS[5]
    k_cpu, v_cpu = workloads.kv_cache()
    k, v = k_cpu.to(dev), v_cpu.to(dev)
    H, T, D = k.shape
    qk, qv = nvfp4.kv_quantize(k), nvfp4.kv_quantize(v)
    ok, ov = torch.empty_like(k), torch.empty_like(v)

    def rt():
        nvfp4.kv_quantize(k, out=qk)
        nvfp4.kv_quantize(v, out=qv)
        nvfp4.kv_dequantize(*qk, out=ok)
        nvfp4.kv_dequantize(*qv, out=ov)

    settle(torch, rt)
    rt_ms = time_calls(torch, rt, steps, warmup)
    _, *rt_pct = time_calls_dist(torch, rt, steps, 0)
    n = 2 * k.numel()
    kb = workloads.bf16_bits(k_cpu[:1])
    t0 = time.perf_counter()
    oc, os_, oh = oracle.kv_quantize(kb)
    oracle.kv_dequantize(oc, os_, oh)
    o_ms = (time.perf_counter() - t0) * 1e3 * 2 * H
    res[c["workload"]] = {"H": H, "T": T, "D": D, "tensors": 2, "roundtrip_ms": round(rt_ms, 4),
                          "roundtrip_ms_p10_p50_p90": rt_pct,
                          "roundtrip_GB/s": round(n * (B_AMAX + B_ENCODE + B_DEQUANT) / (rt_ms * 1e-3) / 1e9, 1),
                          "oracle_roundtrip_ms_est": round(o_ms, 1), "oracle_sample": "1 head of K",
                          "oracle_threads": oracle.num_threads()}
    log("config 5", json.dumps(res[c["workload"]]))
    # attention of a new 4096-query chunk over the packed config-5 cache
    qa_cpu = workloads.attention_queries(H, 4096, D)
    qa = qa_cpu.to(dev)
    Tq = qa.shape[1]
    oa = torch.empty_like(qa)
    wsa = torch.empty(nvfp4.kv_attention_workspace_size(H, Tq, T, D), dtype=torch.uint8, device=dev)
    attn = lambda: nvfp4.kv_attention(qa, qk, qv, out=oa, workspace=wsa)
    settle(torch, attn)
    a_ms = time_calls(torch, attn, steps, warmup)
    flop_a = 4.0 * H * Tq * T * D
    oks = oracle.kv_quantize(workloads.bf16_bits(k_cpu))
    ovs = oracle.kv_quantize(workloads.bf16_bits(v_cpu))
    nq = 4
    t0 = time.perf_counter()
    oracle.kv_attention(workloads.bf16_bits(qa_cpu), oks, ovs, T, D ** -0.5, q_idx=np.arange(nq))
    oa_ms = (time.perf_counter() - t0) * 1e3 * Tq / nq
    res["kv_attention_24x4096_over_65536"] = {
        "H": H, "q_tokens": Tq, "kv_tokens": T, "D": D, "ms": round(a_ms, 4),
        "TFLOP/s": round(flop_a / (a_ms * 1e-3) / 1e12, 1),
        "frac_of_fp16_peak": round(flop_a / (a_ms * 1e-3) / 1e12 / MFMA_PEAK_F16_TFLOPS, 4),
        "workspace_bytes": wsa.numel(), "oracle_ms_est": round(oa_ms, 1),
        "oracle_sample": "%d queries of every head" % nq, "oracle_threads": oracle.num_threads()}
    log("attention", json.dumps(res["kv_attention_24x4096_over_65536"]))
    # RoPE fused into the append: the chunk's 4096 new keys per head rotated into the cache tail
    kn = qa.clone()
    ra = lambda: nvfp4.kv_rope_quantize_append(kn, qk, T - Tq)
    settle(torch, ra, 0.2)
    r_ms_eager = time_calls(torch, ra, steps, warmup)
    r_ms = time_graph(torch, ra)
    nh = 1
    t0 = time.perf_counter()
    yr = oracle.rope(workloads.bf16_bits(qa_cpu[:nh]), np.arange(T - Tq, T), 10000.0)
    oracle.quantize(yr[0], np.float32(oks[2][0]))
    or_ms = (time.perf_counter() - t0) * 1e3 * H / nh
    res["kv_rope_append_24x4096"] = {
        "ms": round(r_ms, 4), "GB/s": round(kn.numel() * (2 + 0.5625) / (r_ms * 1e-3) / 1e9, 1),
        "timing": "HIP graph of 20 calls", "ms_eager": round(r_ms_eager, 4),
        "oracle_ms_est": round(or_ms, 1), "oracle_sample": "%d of %d heads" % (nh, H),
        "oracle_threads": oracle.num_threads()}
    log("rope append", json.dumps(res["kv_rope_append_24x4096"]))
    del kn
    del k, v, qk, qv, ok, ov, qa, oa, wsa, oks, ovs
    torch.cuda.empty_cache()
    # backward of the FFN up-projection: operands quantized along rows, dgrad and wgrad
    a_cpu, w_cpu, dy_cpu = workloads.activations(3), workloads.weights(3), workloads.output_grads(3)
    a, w, dy = a_cpu.to(dev), w_cpu.to(dev), dy_cpu.to(dev)
    dyq, wtq, dytq, atq = nvfp4.quantize(dy), nvfp4.quantize_transposed(w), nvfp4.quantize_transposed(dy), \
        nvfp4.quantize_transposed(a)
    qt = lambda: nvfp4.quantize_transposed(dy, out=dytq[:2], s_g_out=dytq[2])
    settle(torch, qt)
    t_ms = time_calls(torch, qt, steps, warmup)
    dx = nvfp4.gemm(dyq, wtq)
    dw = nvfp4.gemm(dytq, atq)
    dgrad = lambda: nvfp4.gemm(dyq, wtq, out=dx)
    wgrad = lambda: nvfp4.gemm(dytq, atq, out=dw)
    settle(torch, dgrad)
    dx_ms = time_calls(torch, dgrad, steps, warmup)
    dw_ms = time_calls(torch, wgrad, steps, warmup)
    M3, N3 = dy.shape
    K3 = w.shape[1]
    fl = 2.0 * M3 * N3 * K3
    dyn = workloads.bf16_bits(dy_cpu)
    ncol = 256  # oracle: full amax + the columns of one 256-column sample
    t0 = time.perf_counter()
    g = oracle.global_scale(oracle.amax(dyn))
    ta = time.perf_counter()
    oracle.quantize_transposed(np.ascontiguousarray(dyn[:, :ncol]), g)
    t1 = time.perf_counter()
    ot_ms = (ta - t0) * 1e3 + (t1 - ta) * 1e3 * N3 / ncol
    res["backward_ffn_up_16384x14336x3072"] = {
        "quantize_transposed_dY_ms": round(t_ms, 4),
        "quantize_transposed_dY_GB/s": round(dy.numel() * (B_AMAX + B_ENCODE) / (t_ms * 1e-3) / 1e9, 1),
        "dgrad_ms": round(dx_ms, 4), "dgrad_TFLOP/s": round(fl / (dx_ms * 1e-3) / 1e12, 1),
        "wgrad_ms": round(dw_ms, 4), "wgrad_TFLOP/s": round(fl / (dw_ms * 1e-3) / 1e12, 1),
        "oracle_quantize_transposed_ms_est": round(ot_ms, 1),
        "oracle_sample": "full amax, then %d of %d columns" % (ncol, N3), "oracle_threads": oracle.num_threads()}
    log("backward", json.dumps(res["backward_ffn_up_16384x14336x3072"]))
    del a, w, dy, dyq, wtq, dytq, atq, dx, dw
    torch.cuda.empty_cache()
    # adaLN fused into the activation quantizer
    x_cpu, sh_cpu, sc_cpu, rpg = workloads.adaln_inputs()
    xa, sha, sca = x_cpu.to(dev), sh_cpu.to(dev), sc_cpu.to(dev)
    qa_ = nvfp4.adaln_quantize(xa, sha, sca, rpg)
    ada = lambda: nvfp4.adaln_quantize(xa, sha, sca, rpg, out=qa_[:2], s_g_out=qa_[2])
    settle(torch, ada)
    ad_ms = time_calls(torch, ada, steps, warmup)
    nrow = 1024
    xn = workloads.bf16_bits(x_cpu)
    t0 = time.perf_counter()
    yo = oracle.adaln(np.ascontiguousarray(xn[:nrow]), sh_cpu.numpy(), sc_cpu.numpy(), rpg, 1e-6)
    oracle.quantize(yo)
    oad_ms = (time.perf_counter() - t0) * 1e3 * x_cpu.shape[0] / nrow
    res["adaln_quantize_16384x3072"] = {
        "ms": round(ad_ms, 4), "GB/s": round(xa.numel() * B_ADALN / (ad_ms * 1e-3) / 1e9, 1),
        "bytes_per_elem": B_ADALN, "oracle_ms_est": round(oad_ms, 1),
        "oracle_sample": "%d of %d rows (adaLN + quantize)" % (nrow, x_cpu.shape[0]),
        "oracle_threads": oracle.num_threads()}
    log("adaln", json.dumps(res["adaln_quantize_16384x3072"]))
    return res


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn back to back for `seconds` so that the clocks reach steady state."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def cpu_model():
    """The host CPU's model string, family and model numbers (from /proc/cpuinfo;
    virtual machines may shorten the model string)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break  # first processor only
                    continue
                key, val = (t.strip() for t in line.split(":", 1))
                if key in ("model name", "cpu family", "model") and key not in fields:
                    fields[key] = val
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    if "cpu family" in fields and "model" in fields:
        name += " (family %s, model %s)" % (fields["cpu family"], fields["model"])
    return name


def oracle_sample(workloads, rows):
    """The CPU oracle (test infrastructure) on a bounded sample of the step:
    the amax of the whole activation, quantization of its first `rows` rows
    with that scale, and their fp64 reference GEMM rows against all weight
    rows (weights quantized once, not timed).  Returns (seconds, threads)."""
    import numpy as np
    import oracle

    a = workloads.bf16_bits(workloads.activations(3))
    w = workloads.bf16_bits(workloads.weights(3))
    wc, ws, wg = oracle.quantize(w)
    t0 = time.perf_counter()
    g = oracle.global_scale(oracle.amax(a))
    ac, as_, _ = oracle.quantize(np.ascontiguousarray(a[:rows]), s_g=g)
    oracle.gemm_ref(ac, as_, g, wc, ws, wg)
    return time.perf_counter() - t0, oracle.num_threads()


def cpu_baseline(workloads, M, N, K, rows=8192, rows_1t=128):
    """The oracle on the host's cores: all threads on `rows` rows, then one thread
    on `rows_1t` rows, each as TFLOP/s of the same 2 M N K metric scaled by the
    rows it computed."""
    import oracle

    dt, threads = oracle_sample(workloads, rows)
    sample = ("amax of the full A [%d, %d], quantize of its first %%d rows, fp64 reference GEMM of those rows "
              "against all %d weight rows (K = %d)" % (M, K, N, K))
    out = {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "seconds": round(dt, 2), "sample": sample % rows, "cpu_model": cpu_model(),
           "host_cpus": os.cpu_count()}
    oracle.set_num_threads(1)
    try:
        dt1, t1 = oracle_sample(workloads, rows_1t)
    finally:
        oracle.set_num_threads(threads)
    out["single_thread"] = {"value": round(2.0 * rows_1t * N * K / dt1 / 1e12, 6), "cores": t1,
                            "seconds": round(dt1, 2), "sample": sample % rows_1t}
    return out


if __name__ == "__main__":
    main()
