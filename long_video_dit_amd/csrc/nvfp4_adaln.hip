// adaLN fused into the NVFP4 activation quantizer, for gfx950.
//
// The yourai.pro news page lists a unified RoPE + adaLN kernel among the
// NVFP4 inference-path optimizations.  Here the adaLN producer of a linear's
// input is fused into the quantizer of that input, so the modulated
// activation is never written: for row r of x [rows][k] in group
// g = r / rows_per_group,
//   y[r][d] = (x[r][d] - mu_r) * rstd_r * (1 + scale[g][d]) + shift[g][d],
//   mu_r = mean, rstd_r = 1 / sqrt(biased variance + eps), all in fp32,
// and y is quantized to NVFP4 exactly as nvfp4_quantize quantizes a tensor.
// Traffic per element: 2 B (amax pass) + 2 B read + 0.5625 B written, against
// 2 + 2 (adaLN kernel) + 2 (amax) + 2.5625 (encode) for the unfused chain.
//
// One wave per row, the row in registers as loaded (packed bf16): lane l holds
// the 8-element units u = l + 64 j (j < 8, so k <= 4096); lanes 2i and 2i + 1
// hold one 16-element block; y is formed unit by unit where it is used.  The row sums use a six-level tree
// over the wave (every lane ends with the same value, and the order is fixed),
// so the encode pass recomputes exactly the y of the amax pass.
#include <hip/hip_runtime.h>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kRowsPerWg = 4;
constexpr int kMaxJ = 8;  // units per lane: k <= 64 * 8 * 8

// One 8-element unit of x as loaded (bf16: 16 B, fp32: 32 B), kept packed in
// registers; unpacked to fp32 where used.
template <typename T>
struct RawUnit;
template <>
struct RawUnit<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* __restrict__ p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void get(float (&f)[8]) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct RawUnit<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* __restrict__ p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }
  __device__ __forceinline__ void get(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

__device__ __forceinline__ void load8f(const float* __restrict__ p, float (&f)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Sum over the wave, the same value in every lane, in a fixed order: pairs,
// quads, 8 and 16 lanes with DPP moves, then the four 16-lane sums read from
// lanes 0, 16, 32, 48 and added as (r0 + r1) + (r2 + r3).  Six levels, like a
// butterfly, but without LDS round trips (3.5% faster on [16384, 3072]).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Row r held packed by the wave (lane l: units l + 64 j), with its statistics.
template <typename T>
struct AdalnRow {
  RawUnit<T> x[kMaxJ];
  float mu, rstd;
  const float* shg;
  const float* scg;
  int units;

  __device__ __forceinline__ void init(const T* __restrict__ xg, int64_t r, int k, const float* __restrict__ shift,
                                       const float* __restrict__ scale, int64_t g, float eps, int lane) {
    units = k / 8;
    shg = shift + g * k;
    scg = scale + g * k;
    const T* xr = xg + r * k;
#pragma unroll
    for (int j = 0; j < kMaxJ; j++) {
      if (lane + 64 * j < units) x[j].load(xr + 8 * (lane + 64 * j));
      else x[j].zero();
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxJ; j++) {
      float f[8];
      x[j].get(f);
#pragma unroll
      for (int i = 0; i < 8; i++) s += f[i];
    }
    mu = __fdiv_rn(wave_sum(s), (float)k);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxJ; j++) {
      if (lane + 64 * j < units) {
        float f[8];
        x[j].get(f);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float c = f[i] - mu;
          ss = __builtin_fmaf(c, c, ss);
        }
      }
    }
    const float var = __fdiv_rn(wave_sum(ss), (float)k);
    rstd = __fdiv_rn(1.0f, __fsqrt_rn(var + eps));
  }

  // y of unit j of this lane (valid units only).
  __device__ __forceinline__ void y(int j, int lane, float (&out)[8]) const {
    const int u = lane + 64 * j;
    float f[8], b[8], a[8];
    x[j].get(f);
    load8f(shg + 8 * u, b);
    load8f(scg + 8 * u, a);
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = __builtin_fmaf((f[i] - mu) * rstd, 1.0f + a[i], b[i]);
  }
};

// Pass 1: per-workgroup max |y| (fp32 bits: non-negative floats order as integers).
template <typename T>
__global__ __launch_bounds__(64 * kRowsPerWg) void adaln_amax_kernel(const T* __restrict__ x, int64_t rows, int k,
                                                                   const float* __restrict__ shift,
                                                                   const float* __restrict__ scale,
                                                                   int64_t rows_per_group, float eps,
                                                                   uint32_t* __restrict__ partials) {
  __shared__ uint32_t wmax[kRowsPerWg];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerWg + wave;
  float m = 0.0f;
  if (r < rows) {
    AdalnRow<T> row;
    row.init(x, r, k, shift, scale, r / rows_per_group, eps, lane);
#pragma unroll
    for (int j = 0; j < kMaxJ; j++) {
      if (lane + 64 * j < row.units) {
        float y[8];
        row.y(j, lane, y);
#pragma unroll
        for (int i = 0; i < 8; i++) m = __builtin_fmaxf(m, __builtin_fabsf(y[i]));
      }
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, s));
  if (lane == 0) wmax[wave] = __float_as_uint(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wmax[0];
    for (int w = 1; w < kRowsPerWg; w++) b = b > wmax[w] ? b : wmax[w];
    partials[blockIdx.x] = b;
  }
}

// Pass 2: recompute y, encode against s_g.
template <typename T>
__global__ __launch_bounds__(64 * kRowsPerWg) void adaln_encode_kernel(const T* __restrict__ x, int64_t rows, int k,
                                                                     const float* __restrict__ shift,
                                                                     const float* __restrict__ scale,
                                                                     int64_t rows_per_group, float eps,
                                                                     const float* __restrict__ s_g,
                                                                     uint32_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerWg + wave;
  if (r >= rows) return;  // whole wave: no shuffles are left half-done
  const EncodeConsts c = make_encode_consts(s_g[0]);
  AdalnRow<T> row;
  row.init(x, r, k, shift, scale, r / rows_per_group, eps, lane);
  const int units = row.units;
#pragma unroll
  for (int j = 0; j < kMaxJ; j++) {
    if (64 * j >= units) break;  // uniform
    const int u = lane + 64 * j;
    float y[8];
    if (u < units) row.y(j, lane, y);
    else {
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = 0.0f;
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) am = __builtin_fmaxf(am, __builtin_fabsf(y[i]));
    am = pair_max(am);  // the other half of the block (units is even)
    const uint32_t sb = encode_scale(am, c);
    const uint32_t w = encode8(y, sb, c);
    if (u < units) {
      codes[r * units + u] = w;
      if ((lane & 1) == 0) scales[r * (units / 2) + u / 2] = (uint8_t)sb;
    }
  }
}

}  // namespace

hipError_t launch_adaln_quantize(const void* x, int dtype, int64_t rows, int64_t k, const float* shift,
                                 const float* scale, int64_t rows_per_group, float eps, uint8_t* codes,
                                 uint8_t* scales, float* s_g, bool compute_scale, hipStream_t stream) {
  const int64_t wgs = (rows + kRowsPerWg - 1) / kRowsPerWg;
  const bool f32 = dtype == kDtypeF32;
  uint32_t* cw = reinterpret_cast<uint32_t*>(codes);
  hipError_t e = hipSuccess;
  if (compute_scale) {
    if (wgs > 0) {
      // the partials (4 B per workgroup of 4 rows) live in the codes buffer until the encode pass
      e = f32 ? launch_kernel(adaln_amax_kernel<float>, dim3((unsigned)wgs), dim3(64 * kRowsPerWg), 0, stream,
                              (const float*)x, rows, (int)k, shift, scale, rows_per_group, eps, cw)
              : launch_kernel(adaln_amax_kernel<uint16_t>, dim3((unsigned)wgs), dim3(64 * kRowsPerWg), 0, stream,
                              (const uint16_t*)x, rows, (int)k, shift, scale, rows_per_group, eps, cw);
      if (e != hipSuccess) return e;
    }
    e = launch_finalize(cw, (int)wgs, s_g, stream);
    if (e != hipSuccess || wgs == 0) return e;
  }
  if (wgs == 0) return hipSuccess;
  return f32 ? launch_kernel(adaln_encode_kernel<float>, dim3((unsigned)wgs), dim3(64 * kRowsPerWg), 0, stream,
                             (const float*)x, rows, (int)k, shift, scale, rows_per_group, eps, (const float*)s_g, cw,
                             scales)
             : launch_kernel(adaln_encode_kernel<uint16_t>, dim3((unsigned)wgs), dim3(64 * kRowsPerWg), 0, stream,
                             (const uint16_t*)x, rows, (int)k, shift, scale, rows_per_group, eps, (const float*)s_g,
                             cw, scales);
}

}  // namespace nvfp4
