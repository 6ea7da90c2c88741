// Device-side helpers of the gfx950 NVFP4 library: format decode, the exact
// E4M3/E2M1 rounding used by the quantizer, and vector types.
//
// Numeric contract (the pages fix none of it; see include/nvfp4.h): every
// rounding is one round-to-nearest-even of the exact real value.  The fast
// paths below reach that exactly by bracketing: a value is rounded twice by
// the hardware converters (v_cvt_scalef32_pk_fp4_f32 for E2M1,
// v_cvt_pk_fp8_f32 for E4M3FN, both RNE and monotone) from a lower and an
// upper bound of the exact quotient; when both give the same code that code
// is the rounding of the exact quotient.  Otherwise an exact fp64 comparison
// with the midpoint of the two candidates decides (ties to the even code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Relative half-width of the brackets.  The approximate reciprocals below
// carry at most ~2.5 * 2^-23 relative error plus 2^-24 per multiply, far
// inside 2^-18, so [lo, hi] always contains the exact quotient.
constexpr float kBracketLo = 1.0f - 0x1p-18f;
constexpr float kBracketHi = 1.0f + 0x1p-18f;
// Per-tensor scales below this take the exact slow path for every block
// (their reciprocals would leave the fp32 range of the fast path).
constexpr float kTinyScale = 0x1p-100f;

// E4M3FN byte (0..0x7E) -> exact fp32 value.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const float normal = __uint_as_float((b + (120u << 3)) << 20);  // 2^(e-7) * (1 + m/8)
  const float sub = (float)(b & 7u) * 0x1p-9f;                    // 2^-6 * m/8
  return (b >> 3) ? normal : sub;
}

// E2M1 magnitude index (0..7) -> value.
__device__ __forceinline__ float e2m1_mag(uint32_t m) {
  const uint32_t e = m >> 1, f = m & 1u;
  return e ? __builtin_ldexpf(1.0f + 0.5f * (float)f, (int)e - 1) : 0.5f * (float)f;
}

// Hardware RNE conversion of a non-negative ratio to E4M3FN with saturation
// at 448 (the converter itself only saturates up to 464).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float r) {
  const float c = __builtin_fminf(r, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}

// Exact choice between adjacent scale bytes lo < hi = lo + 1 for the ratio
// amax_b / (6 s_g): compare amax_b with midpoint * 6 * s_g in fp64 (the
// product has <= 31 significant bits, the fma result is exact or at least
// correctly signed).  Ties take the even byte.
__device__ __forceinline__ uint32_t scale_pick(float amax_b, float s_g, uint32_t lo, uint32_t hi) {
  const float mid6 = (e4m3_value(lo) + e4m3_value(hi)) * 3.0f;  // exact, <= 7 bits
  const double d = __builtin_fma(-(double)mid6, (double)s_g, (double)amax_b);
  return d > 0.0 ? hi : (d < 0.0 ? lo : ((lo & 1u) ? hi : lo));
}

// Exact E4M3 scale byte from any candidate within one step of the answer.
__device__ __noinline__ uint32_t scale_resolve(float amax_b, float s_g, uint32_t c) {
  if (c < 0x7Eu && scale_pick(amax_b, s_g, c, c + 1) == c + 1) return c + 1;
  if (c > 0u && scale_pick(amax_b, s_g, c - 1, c) == c - 1) return c - 1;
  return c;
}

// Exact choice between adjacent E2M1 magnitudes lo < hi = lo + 1 for
// |x| / (sb_val * s_g).
__device__ __forceinline__ uint32_t mag_pick(float ax, float sb_val, float s_g, uint32_t lo, uint32_t hi) {
  const float c = 0.5f * (e2m1_mag(lo) + e2m1_mag(hi)) * sb_val;  // exact, <= 7 bits
  const double d = __builtin_fma(-(double)c, (double)s_g, (double)ax);
  return d > 0.0 ? hi : (d < 0.0 ? lo : ((lo & 1u) ? hi : lo));
}

// Exact E2M1 code of x from a candidate magnitude within one step.
__device__ __noinline__ uint32_t code_resolve(float x, float sb_val, float s_g, uint32_t m) {
  const float ax = __builtin_fabsf(x);
  if (m < 7u && mag_pick(ax, sb_val, s_g, m, m + 1) == m + 1) m = m + 1;
  else if (m > 0u && mag_pick(ax, sb_val, s_g, m - 1, m) == m - 1) m = m - 1;
  return ((__float_as_uint(x) >> 31) << 3) | m;
}

// max(v, v of lane ^ 1): the block maximum of a lane pair, with one DPP move
// (quad_perm [1, 0, 3, 2]) instead of an LDS permute.
__device__ __forceinline__ float pair_max(float v) {
  return __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
}

// Two fp32 -> one byte of two E2M1 codes (first value in the low nibble),
// written into byte `sel` of `old`.  Scale 1.0: plain RNE with saturation.
#define NVFP4_PK_FP4(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Per-tensor constants of the encoder.
struct EncodeConsts {
  float s_g;
  float i6_lo, i6_hi;  // bracket of 1 / (6 s_g)
  float inv_g;         // ~1 / s_g (within 2^-23)
  int mode;            // 0 fast, 1 all-zero scale (s_g == 0), 2 exact slow path
};

__device__ __forceinline__ EncodeConsts make_encode_consts(float s_g) {
  EncodeConsts c;
  c.s_g = s_g;
  if (!(s_g > 0.0f)) {
    c.mode = 1;
    c.i6_lo = c.i6_hi = c.inv_g = 0.0f;
    return c;
  }
  c.mode = (s_g < kTinyScale) ? 2 : 0;
  const double i6 = 1.0 / (6.0 * (double)s_g);
  c.i6_lo = (float)(i6 * (double)kBracketLo);
  c.i6_hi = (float)(i6 * (double)kBracketHi);
  c.inv_g = (float)(1.0 / (double)s_g);
  return c;
}

// Scale byte of a block with magnitude maximum amax_b.
__device__ __forceinline__ uint32_t encode_scale(float amax_b, const EncodeConsts& c) {
  if (c.mode == 1) return 0u;
  if (c.mode == 2) {
    const double r = (double)amax_b / (6.0 * (double)c.s_g);
    return scale_resolve(amax_b, c.s_g, e4m3_rne_sat((float)r));
  }
  const uint32_t lo = e4m3_rne_sat(amax_b * c.i6_lo);
  const uint32_t hi = e4m3_rne_sat(amax_b * c.i6_hi);
  return lo == hi ? lo : scale_pick(amax_b, c.s_g, lo, hi);
}

// Encode 8 consecutive elements of one block (scale byte sb) into a 32-bit
// word of 8 E2M1 codes, element i in bits 4i+3..4i.
__device__ __forceinline__ uint32_t encode8(const float (&f)[8], uint32_t sb, const EncodeConsts& c) {
  if (c.mode == 1 || sb == 0u) {
    // Zero scale: codes keep only the sign (x * 0 keeps the sign of x).
    uint32_t w = 0;
    w = NVFP4_PK_FP4(w, f[0] * 0.0f, f[1] * 0.0f, 0);
    w = NVFP4_PK_FP4(w, f[2] * 0.0f, f[3] * 0.0f, 1);
    w = NVFP4_PK_FP4(w, f[4] * 0.0f, f[5] * 0.0f, 2);
    w = NVFP4_PK_FP4(w, f[6] * 0.0f, f[7] * 0.0f, 3);
    return w;
  }
  const float sv = e4m3_value(sb);
  if (c.mode == 2) {
    const double S = (double)sv * (double)c.s_g;  // exact
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float y = (float)((double)__builtin_fabsf(f[i]) / S);
      const uint32_t m = (uint32_t)NVFP4_PK_FP4(0u, y, y, 0) & 7u;
      w |= code_resolve(f[i], sv, c.s_g, m) << (4 * i);
    }
    return w;
  }
  const float R = __builtin_amdgcn_rcpf(sv) * c.inv_g;
  const float rl = R * kBracketLo, rh = R * kBracketHi;
  uint32_t wl = 0, wh = 0;
  wl = NVFP4_PK_FP4(wl, f[0] * rl, f[1] * rl, 0);
  wh = NVFP4_PK_FP4(wh, f[0] * rh, f[1] * rh, 0);
  wl = NVFP4_PK_FP4(wl, f[2] * rl, f[3] * rl, 1);
  wh = NVFP4_PK_FP4(wh, f[2] * rh, f[3] * rh, 1);
  wl = NVFP4_PK_FP4(wl, f[4] * rl, f[5] * rl, 2);
  wh = NVFP4_PK_FP4(wh, f[4] * rh, f[5] * rh, 2);
  wl = NVFP4_PK_FP4(wl, f[6] * rl, f[7] * rl, 3);
  wh = NVFP4_PK_FP4(wh, f[6] * rh, f[7] * rh, 3);
  if (__builtin_expect(wl == wh, 1)) return wl;
  // Rare: some element sits within the bracket of an E2M1 midpoint.
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t a = (wl >> (4 * i)) & 7u, b = (wh >> (4 * i)) & 7u;
    uint32_t code = (wl >> (4 * i)) & 15u;
    if (a != b) {
      const uint32_t lo = a < b ? a : b, hi = a < b ? b : a;
      code = ((__float_as_uint(f[i]) >> 31) << 3) | mag_pick(__builtin_fabsf(f[i]), sv, c.s_g, lo, hi);
    }
    w |= code << (4 * i);
  }
  return w;
}

// RN_bf16 of the exact product p * s_g, where p = val(code) * val(scale) is
// exact in fp32 (<= 6 significant bits).  The fp32 product is rounded once
// more by the hardware bf16 conversion; that double rounding can only go
// wrong when the fp32 product is exactly a bf16 midpoint, and then the exact
// fp64 product decides.
__device__ __forceinline__ uint32_t bf16_of_product(float p, float s_g) {
  const float v = p * s_g;
  const uint32_t u = __float_as_uint(v);
  const __bf16 h = (__bf16)v;
  uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, h);
  if (__builtin_expect((u & 0xffffu) == 0x8000u, 0)) {
    const double ex = __builtin_fabs((double)p * (double)s_g);
    const double av = __builtin_fabs((double)v);
    if (ex > av) b = (u >> 16) + 1u;
    else if (ex < av) b = u >> 16;
  }
  return b;
}

}  // namespace nvfp4
