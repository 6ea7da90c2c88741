"""ctypes binding of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: if the library is missing, loading it raises.

The C ABI takes plain pointers and sizes and cannot see a tensor's extent, so
every wrapper here checks each operand's shape, dtype, contiguity and device
against the sizes it derives, and raises ValueError before anything is
launched: a mismatched operand would otherwise become an out-of-bounds device
access.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_LAUNCH, ERR_FLAGS = range(7)
F32, BF16 = 0, 1
SCALE_COMPUTE, SCALE_GIVEN = 0, 1
FOUR_OVER_SIX = 2  # flag bit: FourOverSix block scaling

# Exported names and C signatures, in the order include/nvfp4.h declares them
# (C enums are passed as int).
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
    "nvfp4_gemm_fused_act": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _P, _I, _I, _P]),
    "kv_quantize": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kv_quantize_four_over_six": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kv_quantize_append": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _P]),
    "kv_rope_quantize_append": (_I, [_P, _I64, _I64, _I64, _P, ctypes.c_float, _P, _P, _P, _I64, _I64, _P]),
    "kv_dequantize": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "kv_attention": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P, _P,
                          ctypes.c_size_t, _P]),
    "kv_attention_noalloc": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P,
                                  _P]),
    "kv_attention_workspace_size": (_I, [_I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
}
# NVFP4_NOALLOC_SCRATCH_BYTES: the fixed scratch array of kv_attention_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20

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


_FLOATS = (torch.float32, torch.bfloat16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


class _Operands:
    """Collects a call's tensors: each is checked for its exact shape, dtype and
    contiguity when added; devices are checked last (all on one GPU), so that a
    shape mismatch is reported as such wherever the tensors live."""

    def __init__(self):
        self.ts = []

    def dims(self, t, name, n):
        if not isinstance(t, torch.Tensor) or t.dim() != n:
            raise ValueError("%s must be a %d-D tensor" % (name, n))
        return tuple(int(s) for s in t.shape)

    def want(self, t, name, shape, dtypes):
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a tensor, got %r" % (name, type(t)))
        shape = tuple(int(s) for s in shape)
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if t.dtype not in dtypes:
            raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, " or ".join(str(d) for d in dtypes)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        self.ts.append((name, t))
        return t

    def slot(self, t, name):
        """A one-element fp32 tensor ([1] or a scalar view)."""
        if not isinstance(t, torch.Tensor) or t.numel() != 1:
            raise ValueError("%s must be a one-element float32 tensor" % name)
        return self.want(t, name, tuple(t.shape), _F32)

    def packed(self, rows, k, out, names=("codes", "scales")):
        """Checks caller-provided (codes [rows, k/2], scales [rows, k/16])."""
        if out is not None:
            self.want(out[0], names[0], (rows, k // 2), _U8)
            self.want(out[1], names[1], (rows, k // 16), _U8)

    def operand(self, q, name):
        """An NVFP4 operand (codes [R, K/2], scales [R, K/16], s_g [1]); returns (R, K)."""
        if not isinstance(q, (tuple, list)) or len(q) < 3:
            raise ValueError("%s must be a (codes, scales, s_g) tuple" % name)
        r, half = self.dims(q[0], name + " codes", 2)
        self.want(q[0], name + " codes", (r, half), _U8)
        _k16(2 * half, name + " K")
        self.want(q[1], name + " scales", (r, 2 * half // 16), _U8)
        self.slot(q[2], name + " s_g")
        return r, 2 * half

    def kv_cache(self, cache, name, H, D):
        """An NVFP4 cache (codes [H, T, D/2], scales [H, T, D/16], head_scales [H]); returns T."""
        if not isinstance(cache, (tuple, list)) or len(cache) != 3:
            raise ValueError("%s must be a (codes, scales, head_scales) tuple" % name)
        T = self.dims(cache[0], name + " codes", 3)[1]
        self.want(cache[0], name + " codes", (H, T, D // 2), _U8)
        self.want(cache[1], name + " scales", (H, T, D // 16), _U8)
        self.want(cache[2], name + " head_scales", (H,), _F32)
        return T

    def device(self):
        dev = None
        for name, t in self.ts:
            if not t.is_cuda:
                raise ValueError("%s must be a GPU tensor" % name)
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError("%s is on %s, the other operands on %s" % (name, t.device, dev))
        return dev


def _k16(k, name):
    if k % 16 != 0:
        raise ValueError("%s = %d is not a multiple of 16" % (name, k))


def _alloc_packed(rows, k, out, device):
    if out is not None:
        return out[0], out[1]
    return (torch.empty(rows, k // 2, dtype=torch.uint8, device=device),
            torch.empty(rows, k // 16, dtype=torch.uint8, device=device))


def _scale_arg(ops, s_g, s_g_out):
    """Checks the scale arguments of a quantizer: a given s_g is read (SCALE_GIVEN), else the
    computed one goes to s_g_out (allocated when None).  Returns (flags, tensor or None)."""
    if s_g is not None:
        return SCALE_GIVEN, ops.slot(s_g, "s_g")
    return SCALE_COMPUTE, None if s_g_out is None else ops.slot(s_g_out, "s_g_out")


def _slot_or_new(t, device):
    return torch.empty(1, dtype=torch.float32, device=device) if t is None else t


def quantize(x, s_g=None, out=None, s_g_out=None, four_over_six=False):
    """x [rows, k] (float32/bfloat16, device) -> (codes u8 [rows, k/2], scales u8 [rows, k/16], s_g f32 [1]).

    With s_g given (a device tensor [1]) it is used as is (NVFP4_SCALE_GIVEN);
    otherwise it is computed into s_g_out (allocated when None).  `out` may
    pass preallocated (codes, scales).  four_over_six: FourOverSix block scaling
    (NVFP4_FOUR_OVER_SIX)."""
    ops = _Operands()
    rows, k = ops.dims(x, "x", 2)
    ops.want(x, "x", (rows, k), _FLOATS)
    _k16(k, "k")
    ops.packed(rows, k, out)
    flags, s_g = _scale_arg(ops, s_g, s_g_out)
    dev = ops.device()
    codes, scales = _alloc_packed(rows, k, out, dev)
    s_g = _slot_or_new(s_g, dev)
    if four_over_six:
        flags |= FOUR_OVER_SIX
    _call("nvfp4_quantize", _ptr(x), _dt(x), rows, k, _ptr(codes), _ptr(scales), _ptr(s_g), flags, _stream(dev))
    return codes, scales, s_g


def quantize_transposed(x, s_g=None, out=None, s_g_out=None, four_over_six=False):
    """x [rows, cols] (float32/bfloat16, device) quantized along its rows: the NVFP4 form of x.T,
    (codes u8 [cols, rows/2], scales u8 [cols, rows/16], s_g f32 [1]), without a transposed copy.
    s_g, out, s_g_out and four_over_six as in quantize."""
    ops = _Operands()
    rows, cols = ops.dims(x, "x", 2)
    ops.want(x, "x", (rows, cols), _FLOATS)
    _k16(rows, "rows")
    ops.packed(cols, rows, out)
    flags, s_g = _scale_arg(ops, s_g, s_g_out)
    dev = ops.device()
    codes, scales = _alloc_packed(cols, rows, out, dev)
    s_g = _slot_or_new(s_g, dev)
    if four_over_six:
        flags |= FOUR_OVER_SIX
    _call("nvfp4_quantize_transposed", _ptr(x), _dt(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(s_g), flags,
          _stream(dev))
    return codes, scales, s_g


def adaln_quantize(x, shift, scale, rows_per_group, eps=1e-6, s_g=None, out=None, s_g_out=None):
    """NVFP4 of y = LayerNorm(x) * (1 + scale[g]) + shift[g] (g = row // rows_per_group) without
    writing y: x [rows, k] float32/bfloat16, shift / scale float32 [groups, k] (device), at least
    ceil(rows / rows_per_group) groups.  Returns (codes, scales, s_g) like quantize."""
    ops = _Operands()
    rows, k = ops.dims(x, "x", 2)
    ops.want(x, "x", (rows, k), _FLOATS)
    _k16(k, "k")
    if int(rows_per_group) < 1:
        raise ValueError("rows_per_group must be >= 1")
    groups = (rows + rows_per_group - 1) // rows_per_group
    for t, name in ((shift, "shift"), (scale, "scale")):
        g_ = ops.dims(t, name, 2)[0]
        if g_ < groups:
            raise ValueError("%s has %d groups, %d rows need %d" % (name, g_, rows, groups))
        ops.want(t, name, (g_, k), _F32)
    ops.packed(rows, k, out)
    flags, s_g = _scale_arg(ops, s_g, s_g_out)
    dev = ops.device()
    codes, scales = _alloc_packed(rows, k, out, dev)
    s_g = _slot_or_new(s_g, dev)
    _call("nvfp4_adaln_quantize", _ptr(x), _dt(x), rows, k, _ptr(shift), _ptr(scale), rows_per_group, float(eps),
          _ptr(codes), _ptr(scales), _ptr(s_g), flags, _stream(dev))
    return codes, scales, s_g


def global_scale(x, out=None):
    """Per-tensor scale of x [rows, k] alone: f32 [1] = RN(max|x| / 2688), on the device."""
    ops = _Operands()
    rows, k = ops.dims(x, "x", 2)
    ops.want(x, "x", (rows, k), _FLOATS)
    _k16(k, "k")
    if out is not None:
        ops.slot(out, "out")
    dev = ops.device()
    s_g = _slot_or_new(out, dev)
    _call("nvfp4_global_scale", _ptr(x), _dt(x), rows, k, _ptr(s_g), _stream(dev))
    return s_g


def dequantize(codes, scales, s_g, dtype=torch.bfloat16, out=None):
    """(codes [rows, k/2], scales [rows, k/16], s_g [1]) -> y [rows, k] of `dtype` (or out's)."""
    ops = _Operands()
    rows, k = ops.operand((codes, scales, s_g), "")
    if out is None:
        if dtype not in _FLOATS:
            raise ValueError("dtype must be float32 or bfloat16")
    else:
        ops.want(out, "out", (rows, k), _FLOATS)
    dev = ops.device()
    y = torch.empty(rows, k, dtype=dtype, device=dev) if out is None else out
    _call("nvfp4_dequantize", _ptr(codes), _ptr(scales), _ptr(s_g), rows, k, _ptr(y), _dt(y), _stream(dev))
    return y


def _c_out(ops, out, out_dtype, M, N):
    if out is None:
        if out_dtype not in _FLOATS:
            raise ValueError("out_dtype must be float32 or bfloat16")
    else:
        ops.want(out, "out", (M, N), _FLOATS)


def gemm(a, b, out_dtype=torch.bfloat16, out=None):
    """C = A . B^T for NVFP4 operands a = (codes, scales, s_g) [M, K], b = (...) [N, K]."""
    ops = _Operands()
    M, K = ops.operand(a, "a")
    N, Kb = ops.operand(b, "b")
    if Kb != K:
        raise ValueError("a has K = %d, b has K = %d" % (K, Kb))
    _c_out(ops, out, out_dtype, M, N)
    dev = ops.device()
    ac, as_, ag = a[:3]
    bc, bs, bg = b[:3]
    c = torch.empty(M, N, dtype=out_dtype, device=dev) if out is None else out
    _call("nvfp4_gemm", _ptr(ac), _ptr(as_), _ptr(ag), _ptr(bc), _ptr(bs), _ptr(bg), M, N, K, _ptr(c), _dt(c),
          _stream(dev))
    return c


def gemm_fused_act(a, b, out_dtype=torch.bfloat16, out=None, a_q=None, s_g=None, four_over_six=False):
    """Quantize activations a [M, K] and compute C = A_q . B^T.

    s_g: a device tensor [1] holding the activation scale (e.g. from global_scale), used as
    given (NVFP4_SCALE_GIVEN); None computes it from a.  a_q may pass preallocated
    (codes, scales[, s_g_out]) for the packed activation.  four_over_six: FourOverSix block
    scaling of the activation.  Returns (C, (codes, scales, s_g))."""
    ops = _Operands()
    M, K = ops.dims(a, "a", 2)
    ops.want(a, "a", (M, K), _FLOATS)
    _k16(K, "K")
    N, Kb = ops.operand(b, "b")
    if Kb != K:
        raise ValueError("a has K = %d, b has K = %d" % (K, Kb))
    ops.packed(M, K, None if a_q is None else a_q[:2], ("a_q codes", "a_q scales"))
    flags, sg = _scale_arg(ops, s_g, None if a_q is None or len(a_q) < 3 else a_q[2])
    _c_out(ops, out, out_dtype, M, N)
    dev = ops.device()
    codes, scales = _alloc_packed(M, K, None if a_q is None else a_q[:2], dev)
    sg = _slot_or_new(sg, dev)
    c = torch.empty(M, N, dtype=out_dtype, device=dev) if out is None else out
    bc, bs, bg = b[:3]
    if four_over_six:
        flags |= FOUR_OVER_SIX
    _call("nvfp4_gemm_fused_act", _ptr(a), _dt(a), M, K, _ptr(sg), _ptr(codes), _ptr(scales), _ptr(bc),
          _ptr(bs), _ptr(bg), N, _ptr(c), _dt(c), flags, _stream(dev))
    return c, (codes, scales, sg)


def kv_quantize(kv, out=None, four_over_six=False):
    """kv bf16 [H, T, D] -> (codes [H, T, D/2], scales [H, T, D/16], head_scales f32 [H]);
    four_over_six: FourOverSix block scaling (kv_quantize_four_over_six)."""
    ops = _Operands()
    H, T, D = ops.dims(kv, "kv", 3)
    ops.want(kv, "kv", (H, T, D), _BF16)
    _k16(D, "head_dim")
    if out is not None and ops.kv_cache(out, "out", H, D) != T:
        raise ValueError("out holds %d tokens, kv has %d" % (out[0].shape[1], T))
    dev = ops.device()
    if out is None:
        out = (torch.empty(H, T, D // 2, dtype=torch.uint8, device=dev),
               torch.empty(H, T, D // 16, dtype=torch.uint8, device=dev),
               torch.empty(H, dtype=torch.float32, device=dev))
    _call("kv_quantize_four_over_six" if four_over_six else "kv_quantize", _ptr(kv), H, T, D, _ptr(out[0]),
          _ptr(out[1]), _ptr(out[2]), _stream(dev))
    return out


def kv_quantize_append(kv_new, cache, token_offset):
    """Quantize kv_new bf16 [H, t, D] with the cache's frozen per-head scales into rows
    token_offset .. token_offset + t - 1 of cache = (codes [H, T, D/2], scales [H, T, D/16],
    head_scales f32 [H]), in place.  Returns cache."""
    ops = _Operands()
    H, t, D = ops.dims(kv_new, "kv_new", 3)
    ops.want(kv_new, "kv_new", (H, t, D), _BF16)
    _k16(D, "head_dim")
    T = ops.kv_cache(cache, "cache", H, D)
    if not 0 <= token_offset <= T - t:
        raise ValueError("rows %d .. %d are outside the %d-token cache" % (token_offset, token_offset + t, T))
    dev = ops.device()
    codes, scales, head_scales = cache
    _call("kv_quantize_append", _ptr(kv_new), H, t, D, _ptr(head_scales), _ptr(codes), _ptr(scales),
          T, token_offset, _stream(dev))
    return cache


def kv_dequantize(codes, scales, head_scales, out=None):
    """NVFP4 cache (codes [H, T, D/2], scales [H, T, D/16], head_scales [H]) -> bf16 [H, T, D]."""
    ops = _Operands()
    H, T, half = ops.dims(codes, "codes", 3)
    D = 2 * half
    _k16(D, "head_dim")
    ops.kv_cache((codes, scales, head_scales), "cache", H, D)
    if out is not None:
        ops.want(out, "out", (H, T, D), _BF16)
    dev = ops.device()
    y = torch.empty(H, T, D, dtype=torch.bfloat16, device=dev) if out is None else out
    _call("kv_dequantize", _ptr(codes), _ptr(scales), _ptr(head_scales), H, T, D, _ptr(y), _stream(dev))
    return y


def kv_rope_quantize_append(k_new, cache, token_offset, positions=None, base=10000.0):
    """Rotate new keys k_new bf16 [H, Tn, D] with RoPE (positions int32 [Tn] on the device, default
    token_offset + t) and quantize them in place into rows token_offset .. of the NVFP4 cache
    (codes [H, T, D/2], scales [H, T, D/16], head_scales [H]) under its frozen head scales."""
    ops = _Operands()
    H, Tn, D = ops.dims(k_new, "k_new", 3)
    ops.want(k_new, "k_new", (H, Tn, D), _BF16)
    _k16(D, "head_dim")
    T = ops.kv_cache(cache, "cache", H, D)
    if not 0 <= token_offset <= T - Tn:
        raise ValueError("rows %d .. %d are outside the %d-token cache" % (token_offset, token_offset + Tn, T))
    if positions is not None:
        ops.want(positions, "positions", (Tn,), (torch.int32,))
    dev = ops.device()
    codes, scales, hs = cache
    _call("kv_rope_quantize_append", _ptr(k_new), H, Tn, D, _ptr(positions), float(base), _ptr(hs), _ptr(codes),
          _ptr(scales), T, token_offset, _stream(dev))
    return cache


def kv_attention_workspace_size(heads, q_tokens, kv_tokens, head_dim=128):
    """Workspace bytes at which kv_attention takes its preferred cache split on the current device."""
    n = ctypes.c_size_t(0)
    _call("kv_attention_workspace_size", heads, q_tokens, head_dim, kv_tokens, ctypes.byref(n))
    return n.value


def _attention_args(ops, q, k_cache, v_cache, kv_tokens, scale, out):
    H, Tq, D = ops.dims(q, "q", 3)
    ops.want(q, "q", (H, Tq, D), _BF16)
    T = ops.kv_cache(k_cache, "k_cache", H, D)
    if ops.dims(v_cache[0], "v_cache codes", 3)[1] != T:
        raise ValueError("the K and V caches hold different token counts")
    ops.kv_cache(v_cache, "v_cache", H, D)
    kv_tokens = T if kv_tokens is None else int(kv_tokens)
    if not 1 <= kv_tokens <= T:
        raise ValueError("kv_tokens = %d outside 1 .. %d" % (kv_tokens, T))
    scale = D ** -0.5 if scale is None else float(scale)
    if out is not None:
        ops.want(out, "out", (H, Tq, D), _BF16)
    return H, Tq, D, T, kv_tokens, scale


def kv_attention(q, k_cache, v_cache, kv_tokens=None, scale=None, out=None, workspace=None):
    """Softmax attention of q bf16 [H, Tq, D] over the first kv_tokens rows of the NVFP4 caches
    k_cache, v_cache = (codes [H, T, D/2], scales [H, T, D/16], head_scales [H]); bf16 [H, Tq, D].
    workspace: optional uint8 device tensor for the split-cache partial results (allocated here at
    the preferred size when None; an empty tensor turns the split off)."""
    ops = _Operands()
    H, Tq, D, T, kv_tokens, scale = _attention_args(ops, q, k_cache, v_cache, kv_tokens, scale, out)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        ops.want(workspace, "workspace", (workspace.numel(),), _U8)
    dev = ops.device()
    o = torch.empty_like(q) if out is None else out
    if workspace is None:
        with torch.cuda.device(dev):
            nbytes = kv_attention_workspace_size(H, Tq, kv_tokens, D)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    kc, ks, kh = k_cache
    vc, vs, vh = v_cache
    _call("kv_attention", _ptr(q), H, Tq, D, _ptr(kc), _ptr(ks), _ptr(kh), _ptr(vc), _ptr(vs), _ptr(vh), T, kv_tokens,
          scale, _ptr(o), _ptr(workspace) if workspace.numel() else None, workspace.numel(), _stream(dev))
    return o


def kv_attention_noalloc(q, k_cache, v_cache, kv_tokens=None, scale=None, out=None):
    """kv_attention for callers that cannot allocate: the library's fixed device scratch
    (NOALLOC_SCRATCH_BYTES) holds the split-cache partials; the result equals kv_attention with
    a workspace of that size.  Pass `out` to allocate nothing here either.  Calls that overlap
    in time on one device race (they share the scratch)."""
    ops = _Operands()
    H, Tq, D, T, kv_tokens, scale = _attention_args(ops, q, k_cache, v_cache, kv_tokens, scale, out)
    dev = ops.device()
    o = torch.empty_like(q) if out is None else out
    kc, ks, kh = k_cache
    vc, vs, vh = v_cache
    _call("kv_attention_noalloc", _ptr(q), H, Tq, D, _ptr(kc), _ptr(ks), _ptr(kh), _ptr(vc), _ptr(vs), _ptr(vh), T,
          kv_tokens, scale, _ptr(o), _stream(dev))
    return o
