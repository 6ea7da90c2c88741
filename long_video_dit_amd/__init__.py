"""MI355X (gfx950) NVFP4 hot path of a long-video DiT: block quantization,
dequantization, the W4A4 block-scaled GEMM and the NVFP4 KV cache.

The compute lives in libnvfp4.so (hand-written HIP kernels behind the C ABI
of include/nvfp4.h); ``long_video_dit_amd.nvfp4`` is a thin ctypes binding
that passes torch device pointers and the current HIP stream.
"""
from . import nvfp4  # noqa: F401
