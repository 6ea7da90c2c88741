// Rotary position embedding fused into the NVFP4 KV append, for gfx950.
//
// The yourai.pro news page lists a unified RoPE + adaLN kernel and in-place
// updates of the quantized cache among the NVFP4 inference-path
// optimizations.  Here new keys are rotated and quantized into the packed
// cache in one pass, so the rotated keys never go to HBM in bf16: for head
// h, new token t at position p (positions[t], or token_offset + t) and pair
// i of adjacent dims (2i, 2i + 1),
//   (y_2i, y_2i+1) = (x_2i cos(p th_i) - x_2i+1 sin(p th_i), x_2i sin(p th_i) + x_2i+1 cos(p th_i)),
//   th_i = base^(-2i / D),
// and y is encoded under the frozen per-head scale like kv_quantize_append.
//
// Angles: p * th_i reaches ~6.6e4 rad at 65,536 tokens, where one fp32
// rounding of the angle alone moves it by ~4e-3 rad.  The angle is therefore
// formed and reduced to [-pi, pi] in fp64 (th_i in fp64, Cody-Waite with a
// two-part 2 pi), and only the reduced angle goes to sincosf.
//
// Layout: one lane per 8-element unit of one token, looping over 4 heads
// with that token's sines and cosines (they do not depend on the head); D / 8
// divides 256, so in the grid-stride loop every thread keeps the same unit w
// of head_dim and reads its four th_i once from the workgroup's table.  Lanes
// 2j and 2j + 1 hold one 16-element block.
#include <hip/hip_runtime.h>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeHeads = 4;  // heads per workgroup (blockIdx.y): their loads are issued together
constexpr int kMaxRopePairs = 1024;  // head_dim <= 2048 (head_dim / 8 divides 256)
constexpr double kTwoPiHi = 6.283185307179586232;       // RN_f64(2 pi)
constexpr double kTwoPiLo = 2.4492935982947063545e-16;   // 2 pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189533577;  // only picks the multiple of 2 pi

__global__ __launch_bounds__(kRopeThreads) void rope_encode_kernel(
    const uint16_t* __restrict__ k_new, int heads, int64_t tokens_new, int D, const int32_t* __restrict__ positions,
    int64_t token_offset, double log2_base, const float* __restrict__ head_scales, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t cache_tokens) {
  const int upt = D / 8;  // units per token; divides the stride below
  const int w = threadIdx.x % upt;
  // th_i of the D / 2 pairs, computed once per workgroup rather than four per
  // thread (the fp64 exp2 was ~15% of the kernel's time)
  __shared__ double th_s[kMaxRopePairs];
  for (int i = threadIdx.x; i < D / 2; i += kRopeThreads) th_s[i] = exp2(-(double)(2 * i) / (double)D * log2_base);
  __syncthreads();
  double th[4];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) th[jj] = th_s[4 * w + jj];
  const int64_t units = tokens_new * upt;
  for (int64_t u = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kRopeThreads) {  // pairs of lanes enter and leave together (units even)
    const int64_t t = u / upt;
    const double p = positions ? (double)positions[t] : (double)(token_offset + t);
    float sn[4], cs[4];  // the rotation of this token's unit, shared by every head
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const double ang = p * th[jj];
      const double n = rint(ang * kInvTwoPi);
      const double r = __builtin_fma(-n, kTwoPiLo, __builtin_fma(-n, kTwoPiHi, ang));
      sincosf((float)r, &sn[jj], &cs[jj]);
    }
    const int h0 = blockIdx.y * kRopeHeads;
#pragma unroll
    for (int hh = 0; hh < kRopeHeads; hh++) {
      const int h = h0 + hh;
      if (h >= heads) break;  // uniform
      const EncodeConsts c = make_encode_consts(head_scales[h]);
      const u32x4 v = *reinterpret_cast<const u32x4*>(k_new + ((int64_t)h * tokens_new) * D + 8 * u);
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
      float y[8];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float x0 = __uint_as_float(wd[jj] << 16), x1 = __uint_as_float(wd[jj] & 0xffff0000u);
        y[2 * jj] = __builtin_fmaf(x0, cs[jj], -(x1 * sn[jj]));
        y[2 * jj + 1] = __builtin_fmaf(x0, sn[jj], x1 * cs[jj]);
      }
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) am = __builtin_fmaxf(am, __builtin_fabsf(y[i]));
      am = pair_max(am);
      const uint32_t sb = encode_scale(am, c);
      const int64_t row = (int64_t)h * cache_tokens + token_offset;  // this head's first appended row
      codes[row * upt + u] = encode8(y, sb, c);
      if ((threadIdx.x & 1) == 0) scales[row * (upt / 2) + (u >> 1)] = (uint8_t)sb;
    }
  }
}

}  // namespace

hipError_t launch_kv_rope_append(const void* k_new, int64_t heads, int64_t tokens_new, int64_t head_dim,
                                 const int32_t* positions, double rope_base, const float* head_scales,
                                 uint8_t* codes, uint8_t* scales, int64_t cache_tokens, int64_t token_offset,
                                 hipStream_t stream) {
  if (tokens_new == 0) return hipSuccess;
  const int64_t units = tokens_new * head_dim / 8;
  const int64_t want = (units + kRopeThreads - 1) / kRopeThreads;
  const int64_t hgroups = (heads + kRopeHeads - 1) / kRopeHeads;
  const int64_t cap = std::max<int64_t>(1, (int64_t)device_cu_count() * 16 / hgroups);
  const dim3 grid((unsigned)std::min<int64_t>(want, cap), (unsigned)hgroups);
  return launch_kernel(rope_encode_kernel, grid, dim3(kRopeThreads), 0, stream, (const uint16_t*)k_new, (int)heads,
                       tokens_new, (int)head_dim, positions, token_offset, std::log2(rope_base), head_scales,
                       reinterpret_cast<uint32_t*>(codes), scales, cache_tokens);
}

}  // namespace nvfp4
