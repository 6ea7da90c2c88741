"""ctypes binding of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: if the library is missing, loading it raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_LAUNCH, ERR_FLAGS = range(7)
F32, BF16 = 0, 1
SCALE_COMPUTE, SCALE_GIVEN = 0, 1

# Exported names and C signatures, in the order include/nvfp4.h declares them.
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "nvfp4_abi_version": (_I, []),
    "nvfp4_status_string": (ctypes.c_char_p, [_I]),
    "nvfp4_global_scale": (_I, [_P, _I, _I64, _I64, _P, _P]),
    "nvfp4_quantize": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I, _P]),
    "nvfp4_quantize_transposed": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I, _P]),
    "nvfp4_adaln_quantize": (_I, [_P, _I, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P, _P, _I, _P]),
    "nvfp4_dequantize": (_I, [_P, _P, _P, _I64, _I64, _P, _I, _P]),
    "nvfp4_gemm": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P]),
    "nvfp4_gemm_fused_act": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _P, _I, _P]),
    "kv_quantize": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kv_quantize_append": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _P]),
    "kv_rope_quantize_append": (_I, [_P, _I64, _I64, _I64, _P, ctypes.c_float, _P, _P, _P, _I64, _I64, _P]),
    "kv_dequantize": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "kv_attention": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P, _P,
                          ctypes.c_size_t, _P]),
    "kv_attention_workspace_size": (_I, [_I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
}

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (status %d)" % (fn, lib().nvfp4_status_string(status).decode(), status))
        self.status = status


def lib():
    """The loaded libnvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libnvfp4.so not built: run `python -m long_video_dit_amd.build` "
                              "(or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype, fn.argtypes = res, args
        _lib = l
    return _lib


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != OK:
        raise Nvfp4Error(name, st)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def quantize(x, s_g=None, out=None, s_g_out=None):
    """x [rows, k] (float32/bfloat16, device) -> (codes u8 [rows, k/2], scales u8 [rows, k/16], s_g f32 [1]).

    With s_g given (a device tensor [1]) it is used as is (NVFP4_SCALE_GIVEN);
    otherwise it is computed into s_g_out (allocated when None).  `out` may
    pass preallocated (codes, scales)."""
    _need_cuda(x)
    rows, k = x.shape
    if out is None:
        codes = torch.empty(rows, k // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(rows, k // 16, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    flags = SCALE_COMPUTE if s_g is None else SCALE_GIVEN
    if s_g is None:
        s_g = torch.empty(1, dtype=torch.float32, device=x.device) if s_g_out is None else s_g_out
    _call("nvfp4_quantize", _ptr(x), _dt(x), rows, k, _ptr(codes), _ptr(scales), _ptr(s_g), flags,
          _stream(x.device))
    return codes, scales, s_g


def quantize_transposed(x, s_g=None, out=None, s_g_out=None):
    """x [rows, cols] (float32/bfloat16, device) quantized along its rows: the NVFP4 form of x.T,
    (codes u8 [cols, rows/2], scales u8 [cols, rows/16], s_g f32 [1]), without a transposed copy.
    s_g, out and s_g_out as in quantize."""
    _need_cuda(x)
    rows, cols = x.shape
    if out is None:
        codes = torch.empty(cols, rows // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(cols, rows // 16, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    flags = SCALE_COMPUTE if s_g is None else SCALE_GIVEN
    if s_g is None:
        s_g = torch.empty(1, dtype=torch.float32, device=x.device) if s_g_out is None else s_g_out
    _call("nvfp4_quantize_transposed", _ptr(x), _dt(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(s_g), flags,
          _stream(x.device))
    return codes, scales, s_g


def adaln_quantize(x, shift, scale, rows_per_group, eps=1e-6, s_g=None, out=None, s_g_out=None):
    """NVFP4 of y = LayerNorm(x) * (1 + scale[g]) + shift[g] (g = row // rows_per_group) without
    writing y: x [rows, k] float32/bfloat16, shift / scale float32 [groups, k] (device).
    Returns (codes, scales, s_g) like quantize."""
    _need_cuda(x, shift, scale)
    rows, k = x.shape
    if out is None:
        codes = torch.empty(rows, k // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(rows, k // 16, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    flags = SCALE_COMPUTE if s_g is None else SCALE_GIVEN
    if s_g is None:
        s_g = torch.empty(1, dtype=torch.float32, device=x.device) if s_g_out is None else s_g_out
    _call("nvfp4_adaln_quantize", _ptr(x), _dt(x), rows, k, _ptr(shift), _ptr(scale), rows_per_group, float(eps),
          _ptr(codes), _ptr(scales), _ptr(s_g), flags, _stream(x.device))
    return codes, scales, s_g


def global_scale(x, out=None):
    """Per-tensor scale of x [rows, k] alone: f32 [1] = RN(max|x| / 2688), on the device."""
    _need_cuda(x)
    rows, k = x.shape
    s_g = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    _call("nvfp4_global_scale", _ptr(x), _dt(x), rows, k, _ptr(s_g), _stream(x.device))
    return s_g


def dequantize(codes, scales, s_g, dtype=torch.bfloat16, out=None):
    _need_cuda(codes, scales, s_g)
    rows, k = codes.shape[0], codes.shape[1] * 2
    y = torch.empty(rows, k, dtype=dtype, device=codes.device) if out is None else out
    _call("nvfp4_dequantize", _ptr(codes), _ptr(scales), _ptr(s_g), rows, k, _ptr(y), _dt(y),
          _stream(codes.device))
    return y


def gemm(a, b, out_dtype=torch.bfloat16, out=None):
    """C = A . B^T for NVFP4 operands a = (codes, scales, s_g) [M, K], b = (...) [N, K]."""
    ac, as_, ag = a
    bc, bs, bg = b
    _need_cuda(ac, as_, ag, bc, bs, bg)
    M, K, N = ac.shape[0], ac.shape[1] * 2, bc.shape[0]
    c = torch.empty(M, N, dtype=out_dtype, device=ac.device) if out is None else out
    _call("nvfp4_gemm", _ptr(ac), _ptr(as_), _ptr(ag), _ptr(bc), _ptr(bs), _ptr(bg), M, N, K, _ptr(c), _dt(c),
          _stream(ac.device))
    return c


def gemm_fused_act(a, b, out_dtype=torch.bfloat16, out=None, a_q=None):
    """Quantize activations a [M, K] and compute C = A_q . B^T.

    Returns (C, (a_codes, a_scales, a_sg)); a_q may pass preallocated buffers."""
    _need_cuda(a)
    bc, bs, bg = b
    M, K, N = a.shape[0], a.shape[1], bc.shape[0]
    if a_q is None:
        a_q = (torch.empty(M, K // 2, dtype=torch.uint8, device=a.device),
               torch.empty(M, K // 16, dtype=torch.uint8, device=a.device),
               torch.empty(1, dtype=torch.float32, device=a.device))
    c = torch.empty(M, N, dtype=out_dtype, device=a.device) if out is None else out
    _call("nvfp4_gemm_fused_act", _ptr(a), _dt(a), M, K, _ptr(a_q[2]), _ptr(a_q[0]), _ptr(a_q[1]), _ptr(bc),
          _ptr(bs), _ptr(bg), N, _ptr(c), _dt(c), _stream(a.device))
    return c, a_q


def kv_quantize(kv, out=None):
    """kv bf16 [H, T, D] -> (codes [H, T, D/2], scales [H, T, D/16], head_scales f32 [H])."""
    _need_cuda(kv)
    H, T, D = kv.shape
    if out is None:
        out = (torch.empty(H, T, D // 2, dtype=torch.uint8, device=kv.device),
               torch.empty(H, T, D // 16, dtype=torch.uint8, device=kv.device),
               torch.empty(H, dtype=torch.float32, device=kv.device))
    if kv.dtype != torch.bfloat16:
        raise TypeError("kv_quantize expects bfloat16")
    _call("kv_quantize", _ptr(kv), H, T, D, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream(kv.device))
    return out


def kv_quantize_append(kv_new, cache, token_offset):
    """Quantize kv_new bf16 [H, t, D] with the cache's frozen per-head scales into rows
    token_offset .. token_offset + t - 1 of cache = (codes [H, T, D/2], scales [H, T, D/16],
    head_scales f32 [H]), in place.  Returns cache."""
    _need_cuda(kv_new, *cache)
    H, t, D = kv_new.shape
    codes, scales, head_scales = cache
    _call("kv_quantize_append", _ptr(kv_new), H, t, D, _ptr(head_scales), _ptr(codes), _ptr(scales),
          codes.shape[1], token_offset, _stream(kv_new.device))
    return cache


def kv_dequantize(codes, scales, head_scales, out=None):
    _need_cuda(codes, scales, head_scales)
    H, T, D = codes.shape[0], codes.shape[1], codes.shape[2] * 2
    y = torch.empty(H, T, D, dtype=torch.bfloat16, device=codes.device) if out is None else out
    _call("kv_dequantize", _ptr(codes), _ptr(scales), _ptr(head_scales), H, T, D, _ptr(y), _stream(codes.device))
    return y


def kv_rope_quantize_append(k_new, cache, token_offset, positions=None, base=10000.0):
    """Rotate new keys k_new bf16 [H, Tn, D] with RoPE (positions int32 [Tn] on the device, default
    token_offset + t) and quantize them in place into rows token_offset .. of the NVFP4 cache
    (codes [H, T, D/2], scales [H, T, D/16], head_scales [H]) under its frozen head scales."""
    codes, scales, hs = cache
    _need_cuda(k_new, codes, scales, hs, positions)
    H, Tn, D = k_new.shape
    if positions is not None and positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    _call("kv_rope_quantize_append", _ptr(k_new), H, Tn, D, _ptr(positions), float(base), _ptr(hs), _ptr(codes),
          _ptr(scales), codes.shape[1], token_offset, _stream(k_new.device))
    return cache


def kv_attention_workspace_size(heads, q_tokens, kv_tokens, head_dim=128):
    """Workspace bytes at which kv_attention takes its preferred cache split on the current device."""
    n = ctypes.c_size_t(0)
    _call("kv_attention_workspace_size", heads, q_tokens, head_dim, kv_tokens, ctypes.byref(n))
    return n.value


def kv_attention(q, k_cache, v_cache, kv_tokens=None, scale=None, out=None, workspace=None):
    """Softmax attention of q bf16 [H, Tq, D] over the first kv_tokens rows of the NVFP4 caches
    k_cache, v_cache = (codes [H, T, D/2], scales [H, T, D/16], head_scales [H]); bf16 [H, Tq, D].
    workspace: optional uint8 device tensor for the split-cache partial results (allocated here at
    the preferred size when None; an empty tensor turns the split off)."""
    _need_cuda(q, *k_cache, *v_cache)
    H, Tq, D = q.shape
    kc, ks, kh = k_cache
    vc, vs, vh = v_cache
    T = kc.shape[1]
    kv_tokens = T if kv_tokens is None else kv_tokens
    scale = D ** -0.5 if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    if workspace is None:
        with torch.cuda.device(q.device):
            nbytes = kv_attention_workspace_size(H, Tq, kv_tokens, D)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _need_cuda(workspace)
    _call("kv_attention", _ptr(q), H, Tq, D, _ptr(kc), _ptr(ks), _ptr(kh), _ptr(vc), _ptr(vs), _ptr(vh), T, kv_tokens,
          float(scale), _ptr(o), _ptr(workspace) if workspace.numel() else None, workspace.numel(),
          _stream(q.device))
    return o
