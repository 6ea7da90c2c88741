"""Host-side checks of the built library (no GPU needed): the C ABI exports
every function include/nvfp4.h declares, argument validation rejects bad
calls before any launch, and the GEMM fast path's generated gfx950 assembly
leaves M0 to the direct-to-LDS copies alone."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _lib():
    from long_video_dit_amd import nvfp4
    return nvfp4.lib()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:nvfp4_status_t|int|const char \*)\s*(\w+)\(", text, re.M)))


def test_header_functions_are_exported():
    names = _declared_functions()
    assert set(names) >= {"nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_gemm_fused_act",
                          "kv_quantize", "kv_dequantize", "nvfp4_abi_version", "nvfp4_status_string"}
    lib = _lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\S+)", out))
    assert set(names) <= exported


def test_binding_signatures_cover_header():
    from long_video_dit_amd import nvfp4
    assert set(nvfp4.SIGNATURES) == set(_declared_functions())


def test_version_and_status_strings():
    lib = _lib()
    assert lib.nvfp4_abi_version() == 2
    for st in range(7):
        assert len(lib.nvfp4_status_string(st)) >= 2
    assert lib.nvfp4_status_string(99) == b"unknown status"


def test_validation_errors_launch_nothing():
    """Every invalid-argument path returns its status before touching the GPU."""
    from long_video_dit_amd import nvfp4 as nv
    lib = _lib()
    P = ctypes.c_void_p
    buf = P(1 << 20)  # 16-byte aligned fake address: never dereferenced on these paths
    odd = P((1 << 20) + 2)
    # quantize
    assert lib.nvfp4_quantize(buf, 7, 4, 32, buf, buf, buf, 0, None) == nv.ERR_DTYPE
    assert lib.nvfp4_quantize(buf, 1, 4, 32, buf, buf, buf, 5, None) == nv.ERR_FLAGS
    assert lib.nvfp4_quantize(buf, 1, 4, 32, buf, buf, buf, 4, None) == nv.ERR_FLAGS
    assert lib.nvfp4_quantize(buf, 1, 4, 24, buf, buf, buf, 3, None) == nv.ERR_SHAPE  # 4o6 | given: valid flags
    assert lib.nvfp4_quantize(buf, 1, 4, 24, buf, buf, buf, 0, None) == nv.ERR_SHAPE
    assert lib.nvfp4_quantize(buf, 1, -1, 32, buf, buf, buf, 0, None) == nv.ERR_SHAPE
    assert lib.nvfp4_quantize(buf, 1, 4, 0, buf, buf, buf, 0, None) == nv.ERR_SHAPE
    assert lib.nvfp4_quantize(buf, 1, 1 << 30, 1 << 20, buf, buf, buf, 0, None) == nv.ERR_SHAPE
    assert lib.nvfp4_quantize(None, 1, 4, 32, buf, buf, buf, 0, None) == nv.ERR_NULL
    assert lib.nvfp4_quantize(buf, 1, 4, 32, buf, buf, None, 0, None) == nv.ERR_NULL
    assert lib.nvfp4_quantize(odd, 1, 4, 32, buf, buf, buf, 0, None) == nv.ERR_ALIGN
    # dequantize
    assert lib.nvfp4_global_scale(buf, 2, 4, 32, buf, None) == nv.ERR_DTYPE
    assert lib.nvfp4_global_scale(buf, 1, 4, 40, buf, None) == nv.ERR_SHAPE
    assert lib.nvfp4_global_scale(buf, 1, -2, 32, buf, None) == nv.ERR_SHAPE
    assert lib.nvfp4_global_scale(None, 1, 4, 32, buf, None) == nv.ERR_NULL
    assert lib.nvfp4_global_scale(buf, 1, 4, 32, None, None) == nv.ERR_NULL
    assert lib.nvfp4_global_scale(odd, 0, 4, 32, buf, None) == nv.ERR_ALIGN

    assert lib.nvfp4_dequantize(buf, buf, buf, 4, 32, buf, 3, None) == nv.ERR_DTYPE
    assert lib.nvfp4_dequantize(buf, buf, buf, 4, 40, buf, 1, None) == nv.ERR_SHAPE
    assert lib.nvfp4_dequantize(None, buf, buf, 4, 32, buf, 1, None) == nv.ERR_NULL
    assert lib.nvfp4_dequantize(buf, buf, buf, 4, 32, odd, 1, None) == nv.ERR_ALIGN
    # gemm
    assert lib.nvfp4_gemm(buf, buf, buf, buf, buf, buf, 0, 8, 32, buf, 1, None) == nv.ERR_SHAPE
    assert lib.nvfp4_gemm(buf, buf, buf, buf, buf, buf, 8, 8, 24, buf, 1, None) == nv.ERR_SHAPE
    assert lib.nvfp4_gemm(buf, buf, buf, buf, buf, buf, 1 << 31, 8, 32, buf, 1, None) == nv.ERR_SHAPE
    assert lib.nvfp4_gemm(buf, buf, buf, buf, buf, buf, 8, 8, 32, buf, 9, None) == nv.ERR_DTYPE
    assert lib.nvfp4_gemm(buf, None, buf, buf, buf, buf, 8, 8, 32, buf, 1, None) == nv.ERR_NULL
    assert lib.nvfp4_gemm(buf, buf, buf, odd, buf, buf, 8, 8, 32, buf, 1, None) == nv.ERR_ALIGN
    # fused activation linear
    fa = lib.nvfp4_gemm_fused_act
    assert fa(buf, 5, 8, 32, buf, buf, buf, buf, buf, buf, 8, buf, 1, 0, None) == nv.ERR_DTYPE
    assert fa(buf, 1, 8, 32, buf, buf, buf, buf, buf, buf, 8, buf, 7, 0, None) == nv.ERR_DTYPE  # c dtype
    assert fa(buf, 1, 8, 32, buf, buf, buf, buf, buf, buf, 8, buf, 1, 4, None) == nv.ERR_FLAGS
    assert fa(None, 1, 8, 32, buf, buf, buf, buf, buf, buf, 8, buf, 1, 0, None) == nv.ERR_NULL
    assert fa(buf, 1, 8, 32, None, buf, buf, buf, buf, buf, 8, buf, 1, 1, None) == nv.ERR_NULL  # a_sg, given
    assert fa(buf, 1, 8, 32, buf, None, buf, buf, buf, buf, 8, buf, 1, 0, None) == nv.ERR_NULL  # a_codes
    assert fa(buf, 1, 8, 48 + 8, buf, buf, buf, buf, buf, buf, 8, buf, 1, 0, None) == nv.ERR_SHAPE
    assert fa(odd, 1, 8, 32, buf, buf, buf, buf, buf, buf, 8, buf, 1, 0, None) == nv.ERR_ALIGN
    # KV cache
    assert lib.kv_quantize(buf, 0, 16, 128, buf, buf, buf, None) == nv.ERR_SHAPE
    assert lib.kv_quantize(buf, 4, 16, 120, buf, buf, buf, None) == nv.ERR_SHAPE
    assert lib.kv_quantize(buf, 4, 16, 128, buf, buf, None, None) == nv.ERR_NULL
    assert lib.kv_quantize_append(buf, 4, 16, 128, buf, buf, buf, 64, 49, None) == nv.ERR_SHAPE  # past the cache
    assert lib.kv_quantize_append(buf, 4, 16, 128, buf, buf, buf, 64, -1, None) == nv.ERR_SHAPE
    assert lib.kv_quantize_append(buf, 4, 16, 120, buf, buf, buf, 64, 0, None) == nv.ERR_SHAPE
    assert lib.kv_quantize_append(buf, 4, 16, 128, None, buf, buf, 64, 0, None) == nv.ERR_NULL
    assert lib.kv_quantize_append(None, 4, 16, 128, buf, buf, buf, 64, 0, None) == nv.ERR_NULL
    assert lib.kv_quantize_append(buf, 4, 16, 128, buf, odd, buf, 64, 0, None) == nv.ERR_ALIGN
    assert lib.kv_quantize_append(buf, 4, 0, 128, buf, buf, buf, 64, 64, None) == nv.OK  # empty append
    kva = lambda *a: lib.kv_attention(*a[:-1], None, 0, a[-1])
    assert kva(buf, 2, 8, 64, buf, buf, buf, buf, buf, buf, 32, 32, 0.1, buf, None) == nv.ERR_SHAPE  # head_dim 128
    assert kva(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 33, 0.1, buf, None) == nv.ERR_SHAPE  # > cache
    assert kva(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 0, 0.1, buf, None) == nv.ERR_SHAPE
    assert kva(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 32, float("nan"), buf, None) == nv.ERR_SHAPE
    assert kva(buf, 2, 8, 128, buf, buf, None, buf, buf, buf, 32, 32, 0.1, buf, None) == nv.ERR_NULL
    assert kva(None, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 32, 0.1, buf, None) == nv.ERR_NULL
    assert kva(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 32, 0.1, odd, None) == nv.ERR_ALIGN
    assert lib.kv_attention(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 32, 0.1, buf, odd, 64,
                            None) == nv.ERR_ALIGN  # workspace
    kn = lib.kv_attention_noalloc  # the no-allocation variant validates the same way, before any lookup
    assert kn(buf, 2, 8, 64, buf, buf, buf, buf, buf, buf, 32, 32, 0.1, buf, None) == nv.ERR_SHAPE
    assert kn(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 33, 0.1, buf, None) == nv.ERR_SHAPE
    assert kn(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 32, float("inf"), buf, None) == nv.ERR_SHAPE
    assert kn(buf, 2, 8, 128, buf, buf, buf, None, buf, buf, 32, 32, 0.1, buf, None) == nv.ERR_NULL
    assert kn(buf, 2, 8, 128, buf, buf, buf, buf, buf, buf, 32, 32, 0.1, odd, None) == nv.ERR_ALIGN
    n = ctypes.c_size_t(7)
    assert lib.kv_attention_workspace_size(2, 8, 64, 32, ctypes.byref(n)) == nv.ERR_SHAPE
    assert lib.kv_attention_workspace_size(2, 8, 128, 0, ctypes.byref(n)) == nv.ERR_SHAPE
    assert lib.kv_attention_workspace_size(0, 8, 128, 32, ctypes.byref(n)) == nv.ERR_SHAPE
    assert lib.kv_attention_workspace_size(2, 8, 128, 32, None) == nv.ERR_NULL
    assert n.value == 7
    assert lib.kv_dequantize(buf, buf, buf, 4, -1, 128, buf, None) == nv.ERR_SHAPE
    assert lib.kv_dequantize(buf, buf, buf, 4, 16, 128, odd, None) == nv.ERR_ALIGN
    qt = lib.nvfp4_quantize_transposed
    assert qt(buf, 1, 24, 8, buf, buf, buf, 0, None) == nv.ERR_SHAPE  # rows % 16
    assert qt(buf, 1, 0, 8, buf, buf, buf, 0, None) == nv.ERR_SHAPE
    assert qt(buf, 7, 32, 8, buf, buf, buf, 0, None) == nv.ERR_DTYPE
    assert qt(buf, 1, 32, 8, buf, buf, buf, 5, None) == nv.ERR_FLAGS
    assert qt(None, 1, 32, 8, buf, buf, buf, 0, None) == nv.ERR_NULL
    assert qt(buf, 1, 32, 8, odd, buf, buf, 0, None) == nv.ERR_ALIGN
    ra = lib.kv_rope_quantize_append
    assert ra(buf, 2, 8, 96, None, 1e4, buf, buf, buf, 64, 0, None) == nv.ERR_SHAPE  # 256 % (96 / 8) != 0
    assert ra(buf, 2, 8, 128, None, 0.0, buf, buf, buf, 64, 0, None) == nv.ERR_SHAPE  # base
    assert ra(buf, 2, 8, 128, None, float("nan"), buf, buf, buf, 64, 0, None) == nv.ERR_SHAPE
    assert ra(buf, 2, 8, 128, None, 1e4, buf, buf, buf, 64, 57, None) == nv.ERR_SHAPE  # past the cache
    assert ra(buf, 2, 8, 128, None, 1e4, None, buf, buf, 64, 0, None) == nv.ERR_NULL
    assert ra(buf, 2, 8, 128, odd, 1e4, buf, buf, buf, 64, 0, None) == nv.ERR_ALIGN  # positions
    assert ra(buf, 2, 0, 128, None, 1e4, buf, buf, buf, 64, 64, None) == nv.OK  # empty append
    ad = lib.nvfp4_adaln_quantize
    assert ad(buf, 1, 4, 4112, buf, buf, 2, 1e-6, buf, buf, buf, 0, None) == nv.ERR_SHAPE  # k > 4096
    assert ad(buf, 1, 4, 40, buf, buf, 2, 1e-6, buf, buf, buf, 0, None) == nv.ERR_SHAPE  # k % 16
    assert ad(buf, 1, 4, 64, buf, buf, 0, 1e-6, buf, buf, buf, 0, None) == nv.ERR_SHAPE  # rows_per_group
    assert ad(buf, 1, 1 << 33, 16, buf, buf, 2, 1e-6, buf, buf, buf, 0, None) == nv.ERR_SHAPE  # rows
    assert ad(buf, 1, 4, 64, buf, buf, 2, -1.0, buf, buf, buf, 0, None) == nv.ERR_SHAPE  # eps
    assert ad(buf, 1, 4, 64, buf, buf, 2, float("inf"), buf, buf, buf, 0, None) == nv.ERR_SHAPE
    assert ad(buf, 1, 4, 64, None, buf, 2, 1e-6, buf, buf, buf, 0, None) == nv.ERR_NULL
    assert ad(buf, 1, 4, 64, buf, odd, 2, 1e-6, buf, buf, buf, 0, None) == nv.ERR_ALIGN
    assert ad(buf, 3, 4, 64, buf, buf, 2, 1e-6, buf, buf, buf, 0, None) == nv.ERR_DTYPE
    assert ad(buf, 1, 4, 64, buf, buf, 2, 1e-6, buf, buf, buf, 9, None) == nv.ERR_FLAGS
    assert ad(buf, 1, 4, 64, buf, buf, 2, 1e-6, buf, buf, buf, 2, None) == nv.ERR_FLAGS  # no FourOverSix here
    k46 = lib.kv_quantize_four_over_six
    assert k46(buf, 0, 16, 128, buf, buf, buf, None) == nv.ERR_SHAPE
    assert k46(buf, 4, 16, 120, buf, buf, buf, None) == nv.ERR_SHAPE
    assert k46(buf, 4, 16, 128, buf, buf, None, None) == nv.ERR_NULL
    assert k46(buf, 4, 16, 128, odd, buf, buf, None) == nv.ERR_ALIGN
    assert qt(buf, 1, 32, 8, buf, buf, buf, 6, None) == nv.ERR_FLAGS


def test_attention_split_choice():
    """Host logic of the split-cache attention (a GPU-less host counts 256 CUs,
    as an MI355X has): the workspace it asks for is a whole number of
    per-range partial buffers (fp32 O plus m and l per query, 520 B), none
    when the grid already fills whole rounds of the CUs or the cache is too
    short to cut, and a split when few workgroups would leave CUs idle."""
    from long_video_dit_amd import nvfp4 as nv
    if nv.lib().nvfp4_abi_version() < 1:
        pytest.skip("library too old")
    ws = nv.kv_attention_workspace_size
    per = lambda H, Tq: H * Tq * 520
    assert ws(32, 2048, 65536) == 0          # 8 query blocks x 32 heads = one full round
    assert ws(24, 4096, 200) == 0            # 4 cache blocks: nothing to cut
    assert ws(24, 0, 65536) == 0
    b = ws(24, 256, 65536)                   # 24 workgroups for 256 CUs
    assert b > 0 and b % per(24, 256) == 0 and b // per(24, 256) >= 8
    b = ws(24, 4096, 65536)                  # 384 workgroups: 1.5 rounds unsplit
    assert b > 0 and b % per(24, 4096) == 0
    b = ws(1, 1, 1 << 20)                    # one query, a long cache: split at most 32 ways
    assert 0 < b // per(1, 1) <= 32


_GEMM_ASM = {}


def _gemm_asm():
    """gfx950 assembly of nvfp4_gemm.hip (compiled once per session)."""
    if "asm" not in _GEMM_ASM:
        src = os.path.join(ROOT, "long_video_dit_amd", "csrc", "nvfp4_gemm.hip")
        with tempfile.TemporaryDirectory() as d:
            out = os.path.join(d, "gemm.s")
            r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-device-only", "-O3",
                                "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-S", src,
                                "-o", out], capture_output=True, text=True)
            if r.returncode != 0:
                pytest.fail(r.stderr[-2000:])
            _GEMM_ASM["asm"] = open(out).read()
    return _GEMM_ASM["asm"]


def _fast_kernel_bodies():
    asm = _gemm_asm()
    kernels = re.findall(r"^(_Z\S*fast_kernel\S*):", asm, re.M)
    assert kernels
    return {k: asm[asm.index(k + ":"):asm.index(".Lfunc_end", asm.index(k + ":"))] for k in kernels}


def test_gemm_fast_path_leaves_m0_to_the_lds_copies():
    """The fast GEMM kernel sets M0 inside its own asm statements; the compiler
    must not keep any value of its own in M0 in that kernel."""
    for k, body in _fast_kernel_bodies().items():
        inside = False
        for line in body.splitlines():
            if ";;#ASMSTART" in line:
                inside = True
            elif ";;#ASMEND" in line:
                inside = False
            elif not inside:
                assert not re.search(r"\bm0\b", line.split(";")[0]), (k, line)


def test_gemm_fast_path_accumulators_stay_in_place():
    """The 256 x 256 fast kernels start each tile with zero-accumulator MFMAs
    (an inline 0 as the C operand, chosen in the asm by a scalar compare of an
    SGPR flag) and read the accumulators in place in the epilogue: no
    accumulator zero-writes, no accumulator-to-accumulator copies, and no
    spills, in every fast kernel."""
    bodies = _fast_kernel_bodies()
    for k, body in bodies.items():
        assert "scratch_" not in body, k
        assert not re.search(r"s_cmp_lg_u32 v", body), k  # the flag of the zero-C branch must be an SGPR
        assert len(re.findall(r"v_mfma_f32_32x32x16_f16 a\[\d+:\d+\], v\[\d+:\d+\], v\[\d+:\d+\], 0$", body, re.M)) > 0, k
        assert "v_accvgpr_mov" not in body, k
    full = [k for k in bodies if "Li4E" in k]
    assert len(full) == 2  # bf16 and fp32 output
    for k in full:
        assert "v_accvgpr_write" not in bodies[k], k


def test_binding_rejects_mismatched_operands():
    """The binding checks every operand's shape and dtype against the sizes it
    derives and raises ValueError before any call into the library (CPU
    tensors here: the shape check comes first, the device check last)."""
    import torch
    from long_video_dit_amd import nvfp4 as nv
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    q = lambda r, k: (u8(r, k // 2), u8(r, k // 16), f32(1))
    cases = [
        ("codes", lambda: nv.quantize(bf(8, 64), out=(u8(8, 16), u8(8, 4)))),
        ("scales", lambda: nv.quantize(bf(8, 64), out=(u8(8, 32), u8(8, 5)))),
        ("s_g", lambda: nv.quantize(bf(8, 64), s_g=f32(2))),
        ("dtype", lambda: nv.quantize(torch.zeros(8, 64, dtype=torch.float16))),
        ("multiple of 16", lambda: nv.quantize(bf(8, 40))),
        ("codes", lambda: nv.quantize_transposed(bf(32, 8), out=(u8(32, 16), u8(8, 2)))),
        ("K", lambda: nv.gemm(q(8, 64), q(4, 32))),
        ("b scales", lambda: nv.gemm(q(8, 64), (u8(4, 32), u8(4, 3), f32(1)))),
        ("a s_g", lambda: nv.gemm((u8(8, 32), u8(8, 4), f32(3)), q(4, 64))),
        ("out", lambda: nv.gemm(q(8, 64), q(4, 64), out=f32(4, 8))),
        ("out", lambda: nv.gemm(q(8, 64), q(4, 64), out=torch.zeros(8, 4, dtype=torch.float16))),
        ("K", lambda: nv.gemm_fused_act(bf(8, 64), q(4, 128))),
        ("a_q codes", lambda: nv.gemm_fused_act(bf(8, 64), q(4, 64), a_q=(u8(8, 31), u8(8, 4)))),
        ("s_g", lambda: nv.gemm_fused_act(bf(8, 64), q(4, 64), s_g=f32(1, 2))),
        ("scales", lambda: nv.dequantize(u8(8, 32), u8(8, 3), f32(1))),
        ("out", lambda: nv.dequantize(u8(8, 32), u8(8, 4), f32(1), out=bf(8, 32))),
        ("groups", lambda: nv.adaln_quantize(bf(9, 64), f32(2, 64), f32(3, 64), 4)),
        ("shift", lambda: nv.adaln_quantize(bf(8, 64), f32(2, 48), f32(2, 64), 4)),
        ("shift", lambda: nv.adaln_quantize(bf(8, 64), bf(2, 64), f32(2, 64), 4)),
        ("dtype", lambda: nv.kv_quantize(f32(2, 8, 128))),
        ("out scales", lambda: nv.kv_quantize(bf(2, 8, 128), out=(u8(2, 8, 64), u8(2, 8, 9), f32(2)))),
        ("out head_scales", lambda: nv.kv_quantize(bf(2, 8, 128), out=(u8(2, 8, 64), u8(2, 8, 8), f32(3)))),
        ("cache codes", lambda: nv.kv_quantize_append(bf(2, 4, 128), (u8(2, 16, 32), u8(2, 16, 8), f32(2)), 0)),
        ("cache codes", lambda: nv.kv_quantize_append(bf(2, 4, 128), (u8(3, 16, 64), u8(2, 16, 8), f32(2)), 0)),
        ("outside", lambda: nv.kv_quantize_append(bf(2, 4, 128), (u8(2, 16, 64), u8(2, 16, 8), f32(2)), 13)),
        ("positions", lambda: nv.kv_rope_quantize_append(bf(2, 4, 128), (u8(2, 16, 64), u8(2, 16, 8), f32(2)), 0,
                                                         positions=torch.zeros(4, dtype=torch.int64))),
        ("out", lambda: nv.kv_dequantize(u8(2, 8, 64), u8(2, 8, 8), f32(2), out=bf(2, 8, 64))),
        ("v_cache", lambda: nv.kv_attention(bf(2, 4, 128), (u8(2, 16, 64), u8(2, 16, 8), f32(2)),
                                            (u8(2, 16, 64), u8(2, 15, 8), f32(2)))),
        ("different token counts", lambda: nv.kv_attention(bf(2, 4, 128), (u8(2, 16, 64), u8(2, 16, 8), f32(2)),
                                                           (u8(2, 12, 64), u8(2, 12, 8), f32(2)))),
        ("kv_tokens", lambda: nv.kv_attention(bf(2, 4, 128), (u8(2, 16, 64), u8(2, 16, 8), f32(2)),
                                              (u8(2, 16, 64), u8(2, 16, 8), f32(2)), kv_tokens=17)),
        ("q", lambda: nv.kv_attention(f32(2, 4, 128), (u8(2, 16, 64), u8(2, 16, 8), f32(2)),
                                      (u8(2, 16, 64), u8(2, 16, 8), f32(2)))),
        ("GPU", lambda: nv.quantize(bf(8, 64))),  # right shapes, but host memory
        ("GPU", lambda: nv.gemm(q(8, 64), q(4, 64))),
    ]
    for what, fn in cases:
        with pytest.raises(ValueError, match=what):
            fn()


def test_noalloc_scratch_size_matches_header():
    from long_video_dit_amd import nvfp4 as nv
    m = re.search(r"#define NVFP4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == nv.NOALLOC_SCRATCH_BYTES
