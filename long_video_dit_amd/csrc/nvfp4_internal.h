// Host-side internals shared by the launchers and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <tuple>
#include <utility>

namespace nvfp4 {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// Compute-unit count of the current device (cached per device).
int device_cu_count();

// Launch a kernel through hipLaunchKernel so that the launch status comes back
// directly (no sticky error state is read or cleared).  Arguments are
// converted to the kernel's parameter types before their addresses are taken.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count mismatch");
  std::tuple<P...> t(std::forward<A>(args)...);
  return std::apply(
      [&](auto&... a) {
        void* ptrs[] = {(void*)&a..., nullptr};
        return hipLaunchKernel((const void*)kernel, grid, block, ptrs, shmem, stream);
      },
      t);
}

// Quantizer launchers (nvfp4_quant.hip).  A tensor is `groups` runs of
// units_per_group 8-element units, each run with its own s_g.
hipError_t launch_global_scale(const void* x, int dtype, int64_t units_per_group, int groups, uint32_t* partials,
                               int64_t partial_capacity, float* s_g, hipStream_t stream);
// s_g[0] = RN_f32(max of P partials (fp32 bits) / 2688); P == 0 gives 0.
hipError_t launch_finalize(const uint32_t* partials, int P, float* s_g, hipStream_t stream);
// adaLN of layer-normalized rows fused into the quantizer (nvfp4_adaln.hip),
// k % 16 == 0, k <= 4096.  compute_scale: s_g from the amax of y (partials
// kept in the codes buffer), else the s_g stored at *s_g is used.
hipError_t launch_adaln_quantize(const void* x, int dtype, int64_t rows, int64_t k, const float* shift,
                                 const float* scale, int64_t rows_per_group, float eps, uint8_t* codes,
                                 uint8_t* scales, float* s_g, bool compute_scale, hipStream_t stream);
// RoPE of new keys fused into the NVFP4 KV append (nvfp4_rope.hip), bf16 in,
// 256 % (head_dim / 8) == 0; positions NULL: token_offset + t.
hipError_t launch_kv_rope_append(const void* k_new, int64_t heads, int64_t tokens_new, int64_t head_dim,
                                 const int32_t* positions, double rope_base, const float* head_scales,
                                 uint8_t* codes, uint8_t* scales, int64_t cache_tokens, int64_t token_offset,
                                 hipStream_t stream);
// Standalone per-tensor scale: zero the s_g slot, atomic-max the magnitude
// bits into it, round in place (three kernels, no scratch).
hipError_t launch_global_scale_slot(const void* x, int dtype, int64_t units, float* s_g, hipStream_t stream);
// Encode pass; group g is written at unit g * out_group_stride + out_offset
// (out_group_stride < 0: = units_per_group, a dense tensor).  units_per_group,
// out_group_stride and out_offset must be even (whole 16-element blocks), else
// hipErrorInvalidValue.  four_over_six: FourOverSix block scaling.
hipError_t launch_encode(const void* x, int dtype, int64_t units_per_group, int groups, const float* s_g,
                         uint32_t* codes, uint8_t* scales, hipStream_t stream, int64_t out_group_stride = -1,
                         int64_t out_offset = 0, bool four_over_six = false);
// Encode pass along rows: x [rows][cols] -> NVFP4 of x^T (rows % 16 == 0).
hipError_t launch_encode_t(const void* x, int dtype, int64_t rows, int64_t cols, const float* s_g, uint32_t* codes,
                           uint8_t* scales, hipStream_t stream, bool four_over_six = false);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* s_g, int64_t blocks_per_group,
                          int groups, void* y, int y_dtype, hipStream_t stream);

// Attention over an NVFP4 KV cache (nvfp4_attn.hip), head_dim 128.
hipError_t launch_kv_attention(const void* q, const uint8_t* k_codes, const uint8_t* k_scales, const float* k_hs,
                               const uint8_t* v_codes, const uint8_t* v_scales, const float* v_hs, int64_t heads,
                               int64_t q_tokens, int64_t cache_tokens, int64_t kv_tokens, float scale, void* out,
                               void* workspace, int64_t workspace_bytes, hipStream_t stream);
// The same with the split-cache partials in the library's fixed device array
// (no allocation, no caller workspace).
hipError_t launch_kv_attention_noalloc(const void* q, const uint8_t* k_codes, const uint8_t* k_scales,
                                       const float* k_hs, const uint8_t* v_codes, const uint8_t* v_scales,
                                       const float* v_hs, int64_t heads, int64_t q_tokens, int64_t cache_tokens,
                                       int64_t kv_tokens, float scale, void* out, hipStream_t stream);
// Workspace bytes at which launch_kv_attention takes its preferred cache split
// on the current device (0: no split).
int64_t kv_attention_workspace_bytes(int64_t heads, int64_t q_tokens, int64_t kv_tokens);

// W4A4 GEMM launcher (nvfp4_gemm.hip).
hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_sg, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_sg, int64_t M, int64_t N, int64_t K, void* c,
                       int c_dtype, hipStream_t stream);

}  // namespace nvfp4
