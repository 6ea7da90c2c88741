"""NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, exact CPU reference (``nvfp4_oracle.c``, built with gcc) for
the NVFP4 quantizer, dequantizer, W4A4 GEMM and NVFP4 KV cache.  Only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product library never does, and the two share
no code.  The numeric contract it implements is stated at the top of
``nvfp4_oracle.c`` (E2M1 codes, one E4M3 scale per 16 elements, fp32
per-tensor scale amax/(6*448), every rounding one round-to-nearest-even of the
exact value).  The pages on LongLive-2.0 (arXiv abstract page, Abstract;
d9249.github.io review, "Core idea / structure / operation") name W4A4 NVFP4
linears and an NVFP4 KV cache but fix no numeric detail.

Arrays are numpy: float32 arrays are fp32 tensors, uint16 arrays are bf16
bit patterns.  Every function pinned by the tests in ``tests/test_oracle_*``.
FourOverSix block scaling (``four_over_six=True``) is a reading of a name the
pages give without a definition (d9249.github.io review): its rule is pinned
by exact brute force of that rule, not by the pages.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force=False):
    """Compile nvfp4_oracle.c into liboracle.so (gcc, -O2, no fp contraction)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    c_i64, c_p, c_f, c_d, c_i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_double, ctypes.c_int
    sig = {
        "orc_version": (c_i, []),
        "orc_num_threads": (c_i, []),
        "orc_set_num_threads": (None, [c_i]),
        "orc_e2m1_value": (c_d, [c_i]),
        "orc_e4m3_value": (c_d, [c_i]),
        "orc_global_scale": (c_f, [c_f]),
        "orc_global_scale_f64": (c_f, [c_d]),
        "orc_block_scale": (c_i, [c_d, c_f]),
        "orc_e2m1_code": (c_i, [c_d, c_d]),
        "orc_round_bf16": (ctypes.c_uint16, [c_d]),
        "orc_amax": (c_i, [c_p, c_i, c_i64, c_p]),
        "orc_quantize_with_scale": (c_i, [c_p, c_i, c_i64, c_i64, c_f, c_p, c_p]),
        "orc_quantize": (c_i, [c_p, c_i, c_i64, c_i64, c_p, c_p, c_p]),
        "orc_block_scale4": (c_i, [c_d, c_f]),
        "orc_quantize_4o6_with_scale": (c_i, [c_p, c_i, c_i64, c_i64, c_f, c_p, c_p]),
        "orc_quantize_4o6": (c_i, [c_p, c_i, c_i64, c_i64, c_p, c_p, c_p]),
        "orc_kv_quantize_4o6": (c_i, [c_p, c_i64, c_i64, c_i64, c_p, c_p, c_p]),
        "orc_dequantize": (c_i, [c_p, c_p, c_f, c_i64, c_i64, c_p, c_i]),
        "orc_gemm_ref": (c_i, [c_p, c_p, c_f, c_p, c_p, c_f, c_i64, c_i64, c_i64,
                               c_p, c_i64, c_p, c_i64, c_p, c_p]),
        "orc_kv_quantize": (c_i, [c_p, c_i64, c_i64, c_i64, c_p, c_p, c_p]),
        "orc_adaln": (c_i, [c_p, c_i, c_i64, c_i64, c_p, c_p, c_i64, c_d, c_p]),
        "orc_kv_dequantize": (c_i, [c_p, c_p, c_p, c_i64, c_i64, c_i64, c_p]),
        "orc_kv_attention": (c_i, [c_p, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_d,
                                   c_p, c_i64, c_p, c_p, c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


class OracleError(ValueError):
    pass


def _check(status):
    if status == -1:
        raise OracleError("non-finite input")
    if status != 0:
        raise OracleError("bad shape (status %d)" % status)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.float64:
        return F64
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 / float64 arrays or uint16 bf16 bit patterns, got %s" % x.dtype)


def num_threads():
    return _load().orc_num_threads()


def set_num_threads(n):
    """OpenMP threads of the oracle's loops from now on (results do not depend on it)."""
    _load().orc_set_num_threads(int(n))


# ---- scalar format functions -------------------------------------------

def e2m1_value(code):
    return _load().orc_e2m1_value(int(code))


def e4m3_value(byte):
    return _load().orc_e4m3_value(int(byte))


def global_scale(amax):
    """s_g = RN_f32(amax / 2688) as np.float32."""
    return np.float32(_load().orc_global_scale(float(np.float32(amax))))


def block_scale(amax_b, s_g):
    """E4M3 byte of RNE_SAT(amax_b / (6 s_g))."""
    return _load().orc_block_scale(float(amax_b), float(np.float32(s_g)))


def e2m1_code(x, S):
    """sign | RNE_SAT_E2M1(|x| / S); S = val(s_b) * s_g given exactly."""
    return _load().orc_e2m1_code(float(x), float(S))


def round_bf16(v):
    """bf16 bit pattern of RN_bf16(v) for an exact fp64 value v."""
    return int(_load().orc_round_bf16(float(v)))


# ---- tensors -------------------------------------------------------------

def amax(x):
    x = np.ascontiguousarray(x)
    out = ctypes.c_float(0.0)
    _check(_load().orc_amax(_ptr(x), _dtype_of(x), x.size, ctypes.byref(out)))
    return np.float32(out.value)


def block_scale4(amax_b, s_g):
    """E4M3 byte of RNE_SAT(amax_b / (4 s_g)), the second FourOverSix candidate."""
    return _load().orc_block_scale4(float(amax_b), float(np.float32(s_g)))


def quantize(x, s_g=None, four_over_six=False):
    """x [rows, k] -> (codes uint8 [rows, k/2], scales uint8 [rows, k/16], s_g float32).

    four_over_six: FourOverSix block scaling (a reading: the pages name the backend,
    d9249.github.io review, but do not define it): per block the scale mapping the block
    maximum to 6 or the one mapping it to 4, whichever dequantizes with the smaller exact sum
    of squared errors (ties: 6); s_g as usual."""
    x = np.ascontiguousarray(x)
    if x.ndim != 2:
        raise OracleError("quantize expects a 2-D array")
    rows, k = x.shape
    codes = np.zeros((rows, k // 2), np.uint8)
    scales = np.zeros((rows, k // 16), np.uint8)
    lib = _load()
    full, given = ((lib.orc_quantize_4o6, lib.orc_quantize_4o6_with_scale) if four_over_six else
                   (lib.orc_quantize, lib.orc_quantize_with_scale))
    if s_g is None:
        sg = ctypes.c_float(0.0)
        _check(full(_ptr(x), _dtype_of(x), rows, k, _ptr(codes), _ptr(scales), ctypes.byref(sg)))
        return codes, scales, np.float32(sg.value)
    _check(given(_ptr(x), _dtype_of(x), rows, k, float(np.float32(s_g)), _ptr(codes), _ptr(scales)))
    return codes, scales, np.float32(s_g)


def quantize_transposed(x, s_g=None, four_over_six=False):
    """x [rows, cols] quantized along its rows: the NVFP4 form of x.T, i.e. blocks of 16
    consecutive rows of one column -> (codes [cols, rows/2], scales [cols, rows/16], s_g).
    By definition this is quantize() of the transposed matrix (the pages put NVFP4 on the
    training GEMMs too: landx.limxdynamics.com, sections on NVFP4 and on the training stage;
    d9249.github.io review, "Core idea / structure / operation"); s_g is the same as for x."""
    return quantize(np.ascontiguousarray(np.asarray(x).T), s_g, four_over_six)


def adaln(x, shift, scale, rows_per_group, eps):
    """fp64 y [rows, k] = LayerNorm(x) (no affine, biased variance, eps) * (1 + scale[g]) + shift[g],
    g = row // rows_per_group; x float32 or bf16 bits [rows, k], shift / scale float32 [groups, k].
    The adaLN half of the unified RoPE + adaLN kernel the yourai.pro page lists among the NVFP4
    inference-path optimizations; quantize(y) gives what the fused adaLN quantizer computes."""
    x = np.ascontiguousarray(x)
    rows, k = x.shape
    shift = np.ascontiguousarray(shift, np.float32)
    scale = np.ascontiguousarray(scale, np.float32)
    groups = (rows + rows_per_group - 1) // rows_per_group
    assert shift.shape[0] >= groups and shift.shape[1:] == (k,) and scale.shape == shift.shape
    y = np.empty((rows, k), np.float64)
    _check(_load().orc_adaln(_ptr(x), _dtype_of(x), rows, k, _ptr(shift), _ptr(scale), rows_per_group,
                             float(eps), _ptr(y)))
    return y


def rope(x, positions, base=10000.0):
    """Rotary position embedding of x [H, T, D] (float32 or bf16 bits) in fp64: for every pair of
    adjacent dims (2i, 2i+1) and token t at position p = positions[t],
        (y_2i, y_2i+1) = (x_2i cos(p th_i) - x_2i+1 sin(p th_i), x_2i sin(p th_i) + x_2i+1 cos(p th_i)),
        th_i = base^(-2i / D).
    The RoPE half of the unified RoPE + adaLN kernel the yourai.pro page lists among the NVFP4
    inference-path optimizations; here it rotates new keys before they enter the NVFP4 cache."""
    x = np.asarray(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x
    xf = xf.astype(np.float64)
    H, T, D = xf.shape
    th = np.power(float(base), -np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.asarray(positions, np.float64)[:, None] * th[None, :]
    c, s_ = np.cos(ang)[None], np.sin(ang)[None]
    y = np.empty_like(xf)
    y[..., 0::2] = xf[..., 0::2] * c - xf[..., 1::2] * s_
    y[..., 1::2] = xf[..., 0::2] * s_ + xf[..., 1::2] * c
    return y


def dequantize(codes, scales, s_g, out="bf16"):
    """-> bf16 bit patterns (uint16) or float32 [rows, k]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, k = codes.shape[0], codes.shape[1] * 2
    if out == "bf16":
        y = np.zeros((rows, k), np.uint16)
        dt = BF16
    elif out == "f32":
        y = np.zeros((rows, k), np.float32)
        dt = F32
    else:
        raise ValueError(out)
    _check(_load().orc_dequantize(_ptr(codes), _ptr(scales), float(np.float32(s_g)), rows, k, _ptr(y), dt))
    return y


def gemm_ref(a_codes, a_scales, a_sg, b_codes, b_scales, b_sg, rows=None, cols=None):
    """Reference of C = A . B^T in fp64 and sum_k |a_k b_k| for the selected rows/cols.

    Returns (ref, abssum), float64 arrays [len(rows), len(cols)].
    """
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    a_scales = np.ascontiguousarray(a_scales, np.uint8)
    b_codes = np.ascontiguousarray(b_codes, np.uint8)
    b_scales = np.ascontiguousarray(b_scales, np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    if b_codes.shape[1] * 2 != K:
        raise OracleError("K mismatch")
    r = None if rows is None else np.ascontiguousarray(rows, np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    ref = np.zeros((nr, nc), np.float64)
    tot = np.zeros((nr, nc), np.float64)
    _check(_load().orc_gemm_ref(_ptr(a_codes), _ptr(a_scales), float(np.float32(a_sg)),
                                _ptr(b_codes), _ptr(b_scales), float(np.float32(b_sg)), M, N, K,
                                None if r is None else _ptr(r), nr, None if c is None else _ptr(c), nc,
                                _ptr(ref), _ptr(tot)))
    return ref, tot


def kv_quantize(kv, four_over_six=False):
    """kv bf16 bits uint16 [H, T, D] -> (codes [H,T,D/2], scales [H,T,D/16], head_scales [H]);
    four_over_six as in quantize (per-head scales as usual)."""
    kv = np.ascontiguousarray(kv)
    if kv.dtype != np.uint16 or kv.ndim != 3:
        raise OracleError("kv_quantize expects uint16 bf16 bits [H, T, D]")
    H, T, D = kv.shape
    codes = np.zeros((H, T, D // 2), np.uint8)
    scales = np.zeros((H, T, D // 16), np.uint8)
    hs = np.zeros(H, np.float32)
    fn = _load().orc_kv_quantize_4o6 if four_over_six else _load().orc_kv_quantize
    _check(fn(_ptr(kv), H, T, D, _ptr(codes), _ptr(scales), _ptr(hs)))
    return codes, scales, hs


def kv_dequantize(codes, scales, head_scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    hs = np.ascontiguousarray(head_scales, np.float32)
    H, T, D = codes.shape[0], codes.shape[1], codes.shape[2] * 2
    out = np.zeros((H, T, D), np.uint16)
    _check(_load().orc_kv_dequantize(_ptr(codes), _ptr(scales), _ptr(hs), H, T, D, _ptr(out)))
    return out


def kv_attention(q, k_cache, v_cache, kv_tokens, scale, q_idx=None, return_norm=False):
    """Softmax attention of bf16 queries q (uint16 bits [H, Tq, D]) over the first
    kv_tokens rows of the NVFP4 caches k_cache, v_cache = (codes [H, T, D/2],
    scales [H, T, D/16], head_scales [H]); fp64 on the exact dequantized rows.

    Returns (out, wabs), float64 [H, nq, D]: the attention output and
    sum_j w_j |v_j| / sum_j w_j (q_idx selects the queries of every head); with
    return_norm also the softmax normaliser sum_j w_j [H, nq] (w_j = exp(s_j - max s))."""
    q = np.ascontiguousarray(q)
    if q.dtype != np.uint16 or q.ndim != 3:
        raise OracleError("kv_attention expects uint16 bf16 bits [H, Tq, D]")
    H, Tq, D = q.shape
    kc, ks, kh = (np.ascontiguousarray(a) for a in k_cache)
    vc, vs, vh = (np.ascontiguousarray(a) for a in v_cache)
    T = kc.shape[1]
    kh = np.ascontiguousarray(kh, np.float32)
    vh = np.ascontiguousarray(vh, np.float32)
    qi = None if q_idx is None else np.ascontiguousarray(q_idx, np.int64)
    nq = Tq if qi is None else qi.size
    out = np.zeros((H, nq, D), np.float64)
    wabs = np.zeros((H, nq, D), np.float64)
    lsum = np.zeros((H, nq), np.float64)
    _check(_load().orc_kv_attention(_ptr(q), H, Tq, D, _ptr(kc), _ptr(ks), _ptr(kh), _ptr(vc), _ptr(vs), _ptr(vh),
                                    T, kv_tokens, float(scale), None if qi is None else _ptr(qi), nq,
                                    _ptr(out), _ptr(wabs), _ptr(lsum)))
    return (out, wabs, lsum) if return_norm else (out, wabs)
