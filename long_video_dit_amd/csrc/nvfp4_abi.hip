// C ABI of the NVFP4 library (include/nvfp4.h): argument validation, then
// kernel launches on the caller's stream.  Nothing here allocates, copies,
// synchronizes or reads device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/nvfp4.h"
#include "nvfp4_internal.h"

#include <cmath>

namespace nvfp4 {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace nvfp4

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_dtype(int d) { return d == nvfp4::kDtypeF32 || d == nvfp4::kDtypeBf16; }

// rows x k with k % 16 == 0, within the size limit.
nvfp4_status_t check_matrix(int64_t rows, int64_t k, bool rows_may_be_zero) {
  if (rows < 0 || (rows == 0 && !rows_may_be_zero) || k <= 0 || k % 16 != 0) return NVFP4_ERR_SHAPE;
  if (k > kMaxElems || (rows > 0 && rows > kMaxElems / k)) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

nvfp4_status_t from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

// flags of the quantizing calls: a scale mode, optionally | NVFP4_FOUR_OVER_SIX.
bool valid_flags(int flags, bool four_over_six_allowed) {
  const int extra = four_over_six_allowed ? NVFP4_FOUR_OVER_SIX : 0;
  return (flags & ~(NVFP4_SCALE_GIVEN | extra)) == 0;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(nvfp4_status_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (sizes must be positive, k a multiple of 16, within limits)";
    case NVFP4_ERR_ALIGN: return "misaligned pointer (data 16-byte, scales and s_g 4-byte aligned)";
    case NVFP4_ERR_DTYPE: return "unknown dtype";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    case NVFP4_ERR_FLAGS: return "unknown flags";
    default: return "unknown status";
  }
}

nvfp4_status_t nvfp4_global_scale(const void* x, nvfp4_dtype_t dtype, int64_t rows, int64_t k, float* s_g, void* stream) {
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  nvfp4_status_t st = check_matrix(rows, k, true);
  if (st != NVFP4_OK) return st;
  if (!s_g || (rows > 0 && !x)) return NVFP4_ERR_NULL;
  if (!aligned(s_g, 4) || !aligned(x, 16)) return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_global_scale_slot(x, dtype, rows * k / 8, s_g, (hipStream_t)stream));
}

nvfp4_status_t nvfp4_quantize(const void* x, nvfp4_dtype_t dtype, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales,
                              float* s_g, int flags, void* stream) {
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  if (!valid_flags(flags, true)) return NVFP4_ERR_FLAGS;
  nvfp4_status_t st = check_matrix(rows, k, true);
  if (st != NVFP4_OK) return st;
  if (!s_g || (rows > 0 && (!x || !codes || !scales))) return NVFP4_ERR_NULL;
  if (!aligned(s_g, 4) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t units = rows * k / 8;
  if (!(flags & NVFP4_SCALE_GIVEN)) {
    st = from_hip(nvfp4::launch_global_scale(x, dtype, units, 1, reinterpret_cast<uint32_t*>(codes), units, s_g, s));
    if (st != NVFP4_OK) return st;
  }
  return from_hip(nvfp4::launch_encode(x, dtype, units, 1, s_g, reinterpret_cast<uint32_t*>(codes), scales, s, -1, 0,
                                       (flags & NVFP4_FOUR_OVER_SIX) != 0));
}

nvfp4_status_t nvfp4_quantize_transposed(const void* x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols, uint8_t* codes_t,
                                         uint8_t* scales_t, float* s_g, int flags, void* stream) {
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  if (!valid_flags(flags, true)) return NVFP4_ERR_FLAGS;
  nvfp4_status_t st = check_matrix(cols, rows, true);  // x^T is [cols][rows], blocks along rows
  if (st != NVFP4_OK) return st;
  if (!s_g || (cols > 0 && (!x || !codes_t || !scales_t))) return NVFP4_ERR_NULL;
  if (!aligned(s_g, 4) || !aligned(x, 16) || !aligned(codes_t, 16) || !aligned(scales_t, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t units = rows * cols / 8;
  if (!(flags & NVFP4_SCALE_GIVEN)) {
    st = from_hip(nvfp4::launch_global_scale(x, dtype, units, 1, reinterpret_cast<uint32_t*>(codes_t), units, s_g, s));
    if (st != NVFP4_OK) return st;
  }
  return from_hip(nvfp4::launch_encode_t(x, dtype, rows, cols, s_g, reinterpret_cast<uint32_t*>(codes_t), scales_t, s,
                                         (flags & NVFP4_FOUR_OVER_SIX) != 0));
}

nvfp4_status_t nvfp4_adaln_quantize(const void* x, nvfp4_dtype_t dtype, int64_t rows, int64_t k, const float* shift,
                                    const float* scale, int64_t rows_per_group, float eps, uint8_t* codes,
                                    uint8_t* scales, float* s_g, int flags, void* stream) {
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  if (!valid_flags(flags, false)) return NVFP4_ERR_FLAGS;
  nvfp4_status_t st = check_matrix(rows, k, true);
  if (st != NVFP4_OK) return st;
  // one workgroup per 4 rows: the grid and the partial count stay below 2^31
  if (k > 4096 || rows >= (int64_t(1) << 33) || rows_per_group <= 0 || !std::isfinite(eps) || !(eps >= 0.0f))
    return NVFP4_ERR_SHAPE;
  if (!s_g || (rows > 0 && (!x || !codes || !scales || !shift || !scale))) return NVFP4_ERR_NULL;
  if (!aligned(s_g, 4) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(shift, 16) ||
      !aligned(scale, 16))
    return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_adaln_quantize(x, dtype, rows, k, shift, scale, rows_per_group, eps, codes, scales,
                                               s_g, flags == NVFP4_SCALE_COMPUTE, (hipStream_t)stream));
}

nvfp4_status_t nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s_g, int64_t rows,
                                int64_t k, void* y, nvfp4_dtype_t y_dtype, void* stream) {
  if (!valid_dtype(y_dtype)) return NVFP4_ERR_DTYPE;
  nvfp4_status_t st = check_matrix(rows, k, true);
  if (st != NVFP4_OK) return st;
  if (!s_g || (rows > 0 && (!codes || !scales || !y))) return NVFP4_ERR_NULL;
  if (!aligned(s_g, 4) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_dequant(codes, scales, s_g, rows * k / 16, 1, y, y_dtype, (hipStream_t)stream));
}

static nvfp4_status_t check_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_sg,
                                 const uint8_t* b_codes, const uint8_t* b_scales, const float* b_sg, int64_t M,
                                 int64_t N, int64_t K, const void* c, int c_dtype) {
  if (!valid_dtype(c_dtype)) return NVFP4_ERR_DTYPE;
  if (M <= 0 || N <= 0 || M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31))
    return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_matrix(M, K, false);
  if (st == NVFP4_OK) st = check_matrix(N, K, false);
  if (st == NVFP4_OK && M > kMaxElems / N) st = NVFP4_ERR_SHAPE;
  if (st != NVFP4_OK) return st;
  if (!a_codes || !a_scales || !a_sg || !b_codes || !b_scales || !b_sg || !c) return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
      !aligned(a_sg, 4) || !aligned(b_sg, 4) || !aligned(c, 16))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

nvfp4_status_t nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_sg, const uint8_t* b_codes,
                          const uint8_t* b_scales, const float* b_sg, int64_t M, int64_t N, int64_t K, void* c,
                          nvfp4_dtype_t c_dtype, void* stream) {
  nvfp4_status_t st = check_gemm(a_codes, a_scales, a_sg, b_codes, b_scales, b_sg, M, N, K, c, c_dtype);
  if (st != NVFP4_OK) return st;
  return from_hip(nvfp4::launch_gemm(a_codes, a_scales, a_sg, b_codes, b_scales, b_sg, M, N, K, c, c_dtype,
                                     (hipStream_t)stream));
}

nvfp4_status_t nvfp4_gemm_fused_act(const void* a, nvfp4_dtype_t a_dtype, int64_t M, int64_t K, float* a_sg,
                                    uint8_t* a_codes, uint8_t* a_scales, const uint8_t* b_codes,
                                    const uint8_t* b_scales, const float* b_sg, int64_t N, void* c,
                                    nvfp4_dtype_t c_dtype, int flags, void* stream) {
  if (!valid_dtype(a_dtype)) return NVFP4_ERR_DTYPE;
  if (!valid_flags(flags, true)) return NVFP4_ERR_FLAGS;
  nvfp4_status_t st = check_gemm(a_codes, a_scales, a_sg, b_codes, b_scales, b_sg, M, N, K, c, c_dtype);
  if (st != NVFP4_OK) return st;
  if (!a) return NVFP4_ERR_NULL;
  if (!aligned(a, 16)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t units = M * K / 8;
  if (!(flags & NVFP4_SCALE_GIVEN)) {
    st = from_hip(
        nvfp4::launch_global_scale(a, a_dtype, units, 1, reinterpret_cast<uint32_t*>(a_codes), units, a_sg, s));
    if (st != NVFP4_OK) return st;
  }
  st = from_hip(nvfp4::launch_encode(a, a_dtype, units, 1, a_sg, reinterpret_cast<uint32_t*>(a_codes), a_scales, s,
                                     -1, 0, (flags & NVFP4_FOUR_OVER_SIX) != 0));
  if (st != NVFP4_OK) return st;
  return from_hip(nvfp4::launch_gemm(a_codes, a_scales, a_sg, b_codes, b_scales, b_sg, M, N, K, c, c_dtype, s));
}

static nvfp4_status_t check_kv(int64_t heads, int64_t tokens, int64_t head_dim) {
  if (heads <= 0 || heads > 65535 || tokens < 0 || head_dim <= 0 || head_dim % 16 != 0) return NVFP4_ERR_SHAPE;
  if (head_dim > kMaxElems || tokens > kMaxElems / head_dim || heads > kMaxElems / (tokens * head_dim + 1))
    return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

static nvfp4_status_t kv_quantize_impl(const void* kv, int64_t heads, int64_t tokens, int64_t head_dim,
                                       uint8_t* codes, uint8_t* scales, float* head_scales, bool four_over_six,
                                       void* stream) {
  nvfp4_status_t st = check_kv(heads, tokens, head_dim);
  if (st != NVFP4_OK) return st;
  if (!head_scales || (tokens > 0 && (!kv || !codes || !scales))) return NVFP4_ERR_NULL;
  if (!aligned(head_scales, 4) || !aligned(kv, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t units = tokens * head_dim / 8;
  st = from_hip(nvfp4::launch_global_scale(kv, nvfp4::kDtypeBf16, units, (int)heads,
                                           reinterpret_cast<uint32_t*>(codes), units * heads, head_scales, s));
  if (st != NVFP4_OK) return st;
  return from_hip(nvfp4::launch_encode(kv, nvfp4::kDtypeBf16, units, (int)heads, head_scales,
                                       reinterpret_cast<uint32_t*>(codes), scales, s, -1, 0, four_over_six));
}

nvfp4_status_t kv_quantize(const void* kv, int64_t heads, int64_t tokens, int64_t head_dim, uint8_t* codes,
                           uint8_t* scales, float* head_scales, void* stream) {
  return kv_quantize_impl(kv, heads, tokens, head_dim, codes, scales, head_scales, false, stream);
}

nvfp4_status_t kv_quantize_four_over_six(const void* kv, int64_t heads, int64_t tokens, int64_t head_dim,
                                         uint8_t* codes, uint8_t* scales, float* head_scales, void* stream) {
  return kv_quantize_impl(kv, heads, tokens, head_dim, codes, scales, head_scales, true, stream);
}

nvfp4_status_t kv_quantize_append(const void* kv_new, int64_t heads, int64_t tokens_new, int64_t head_dim,
                                  const float* head_scales, uint8_t* codes, uint8_t* scales, int64_t cache_tokens,
                                  int64_t token_offset, void* stream) {
  nvfp4_status_t st = check_kv(heads, tokens_new, head_dim);
  if (st == NVFP4_OK) st = check_kv(heads, cache_tokens, head_dim);
  if (st != NVFP4_OK) return st;
  if (token_offset < 0 || token_offset > cache_tokens || tokens_new > cache_tokens - token_offset) return NVFP4_ERR_SHAPE;
  if (!head_scales || (tokens_new > 0 && (!kv_new || !codes || !scales))) return NVFP4_ERR_NULL;
  if (!aligned(head_scales, 4) || !aligned(kv_new, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return NVFP4_ERR_ALIGN;
  if (tokens_new == 0) return NVFP4_OK;
  const int64_t units_new = tokens_new * head_dim / 8;  // 8-element units of one head's new rows
  return from_hip(nvfp4::launch_encode(kv_new, nvfp4::kDtypeBf16, units_new, (int)heads, head_scales,
                                       reinterpret_cast<uint32_t*>(codes), scales, (hipStream_t)stream,
                                       cache_tokens * head_dim / 8, token_offset * head_dim / 8));
}

nvfp4_status_t kv_rope_quantize_append(const void* k_new, int64_t heads, int64_t tokens_new, int64_t head_dim,
                                       const int32_t* positions, float rope_base, const float* head_scales,
                                       uint8_t* codes, uint8_t* scales, int64_t cache_tokens, int64_t token_offset,
                                       void* stream) {
  nvfp4_status_t st = check_kv(heads, tokens_new, head_dim);
  if (st == NVFP4_OK) st = check_kv(heads, cache_tokens, head_dim);
  if (st != NVFP4_OK) return st;
  if (256 % (head_dim / 8) != 0 || !std::isfinite(rope_base) || !(rope_base > 0.0f)) return NVFP4_ERR_SHAPE;
  if (token_offset < 0 || token_offset > cache_tokens || tokens_new > cache_tokens - token_offset) return NVFP4_ERR_SHAPE;
  if (!head_scales || (tokens_new > 0 && (!k_new || !codes || !scales))) return NVFP4_ERR_NULL;
  if (!aligned(head_scales, 4) || !aligned(k_new, 16) || !aligned(codes, 16) || !aligned(scales, 4) ||
      !aligned(positions, 4))
    return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_kv_rope_append(k_new, heads, tokens_new, head_dim, positions, (double)rope_base,
                                               head_scales, codes, scales, cache_tokens, token_offset,
                                               (hipStream_t)stream));
}

nvfp4_status_t kv_dequantize(const uint8_t* codes, const uint8_t* scales, const float* head_scales, int64_t heads,
                             int64_t tokens, int64_t head_dim, void* kv_out, void* stream) {
  nvfp4_status_t st = check_kv(heads, tokens, head_dim);
  if (st != NVFP4_OK) return st;
  if (!head_scales || (tokens > 0 && (!codes || !scales || !kv_out))) return NVFP4_ERR_NULL;
  if (!aligned(head_scales, 4) || !aligned(kv_out, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_dequant(codes, scales, head_scales, tokens * head_dim / 16, (int)heads, kv_out,
                                        nvfp4::kDtypeBf16, (hipStream_t)stream));
}

nvfp4_status_t kv_attention_workspace_size(int64_t heads, int64_t q_tokens, int64_t head_dim, int64_t kv_tokens,
                                           size_t* bytes) {
  if (!bytes) return NVFP4_ERR_NULL;
  if (head_dim != 128 || heads <= 0 || heads > 65535 || q_tokens < 0 || q_tokens >= (int64_t(1) << 31) ||
      kv_tokens <= 0 || kv_tokens >= (int64_t(1) << 31) || (q_tokens > 0 && heads > kMaxElems / (q_tokens * head_dim)))
    return NVFP4_ERR_SHAPE;
  *bytes = (size_t)nvfp4::kv_attention_workspace_bytes(heads, q_tokens, kv_tokens);
  return NVFP4_OK;
}

static nvfp4_status_t check_attention(const void* q, int64_t heads, int64_t q_tokens, int64_t head_dim,
                                      const uint8_t* k_codes, const uint8_t* k_scales, const float* k_head_scales,
                                      const uint8_t* v_codes, const uint8_t* v_scales, const float* v_head_scales,
                                      int64_t cache_tokens, int64_t kv_tokens, float softmax_scale, const void* out) {
  if (head_dim != 128 || heads <= 0 || heads > 65535 || q_tokens < 0 || q_tokens >= (int64_t(1) << 31) ||
      kv_tokens <= 0 || kv_tokens > cache_tokens || cache_tokens >= (int64_t(1) << 31) ||
      heads > kMaxElems / (cache_tokens * head_dim) || (q_tokens > 0 && heads > kMaxElems / (q_tokens * head_dim)) ||
      !std::isfinite(softmax_scale))
    return NVFP4_ERR_SHAPE;
  if (!k_head_scales || !v_head_scales || !k_codes || !k_scales || !v_codes || !v_scales ||
      (q_tokens > 0 && (!q || !out)))
    return NVFP4_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(k_head_scales, 4) || !aligned(v_head_scales, 4))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

nvfp4_status_t kv_attention(const void* q, int64_t heads, int64_t q_tokens, int64_t head_dim, const uint8_t* k_codes,
                            const uint8_t* k_scales, const float* k_head_scales, const uint8_t* v_codes,
                            const uint8_t* v_scales, const float* v_head_scales, int64_t cache_tokens,
                            int64_t kv_tokens, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  nvfp4_status_t st = check_attention(q, heads, q_tokens, head_dim, k_codes, k_scales, k_head_scales, v_codes,
                                      v_scales, v_head_scales, cache_tokens, kv_tokens, softmax_scale, out);
  if (st != NVFP4_OK) return st;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  const int64_t ws = workspace ? (int64_t)std::min<size_t>(workspace_bytes, (size_t)INT64_MAX) : 0;
  return from_hip(nvfp4::launch_kv_attention(q, k_codes, k_scales, k_head_scales, v_codes, v_scales, v_head_scales,
                                             heads, q_tokens, cache_tokens, kv_tokens, softmax_scale, out, workspace,
                                             ws, (hipStream_t)stream));
}

nvfp4_status_t kv_attention_noalloc(const void* q, int64_t heads, int64_t q_tokens, int64_t head_dim,
                                    const uint8_t* k_codes, const uint8_t* k_scales, const float* k_head_scales,
                                    const uint8_t* v_codes, const uint8_t* v_scales, const float* v_head_scales,
                                    int64_t cache_tokens, int64_t kv_tokens, float softmax_scale, void* out,
                                    void* stream) {
  nvfp4_status_t st = check_attention(q, heads, q_tokens, head_dim, k_codes, k_scales, k_head_scales, v_codes,
                                      v_scales, v_head_scales, cache_tokens, kv_tokens, softmax_scale, out);
  if (st != NVFP4_OK) return st;
  return from_hip(nvfp4::launch_kv_attention_noalloc(q, k_codes, k_scales, k_head_scales, v_codes, v_scales,
                                                     v_head_scales, heads, q_tokens, cache_tokens, kv_tokens,
                                                     softmax_scale, out, (hipStream_t)stream));
}

}  // extern "C"
