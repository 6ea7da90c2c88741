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
  float i4_lo, i4_hi;  // bracket of 1 / (4 s_g) (FourOverSix's second candidate)
  float inv_g;         // ~1 / s_g (within 2^-23)
  float g_norm;        // s_g 2^-g_exp, in [1, 2) (exact)
  int g_exp;
  int mode;            // 0 fast, 1 all-zero scale (s_g == 0), 2 exact slow path
};

__device__ __forceinline__ EncodeConsts make_encode_consts(float s_g) {
  EncodeConsts c;
  c.s_g = s_g;
  if (!(s_g > 0.0f)) {
    c.mode = 1;
    c.i6_lo = c.i6_hi = c.i4_lo = c.i4_hi = c.inv_g = c.g_norm = 0.0f;
    c.g_exp = 0;
    return c;
  }
  int e;
  (void)__builtin_frexpf(s_g, &e);  // s_g = m 2^e, m in [0.5, 1)
  c.g_exp = e - 1;
  c.g_norm = __builtin_ldexpf(s_g, -c.g_exp);
  c.mode = (s_g < kTinyScale) ? 2 : 0;
  // fp32 reciprocals (v_rcp_f32, within 1 ulp; 6 s_g and 4 s_g round by at
  // most half an ulp, the bracket products by another): each bracket end is
  // off by under 2^-21 relative, far inside its 2^-18 margin, so lo stays
  // below and hi above the exact reciprocal.  In the tiny-scale mode these
  // are unused (they may overflow there).
  const float i6 = __builtin_amdgcn_rcpf(6.0f * s_g), i4 = __builtin_amdgcn_rcpf(4.0f * s_g);
  c.i6_lo = i6 * kBracketLo;
  c.i6_hi = i6 * kBracketHi;
  c.i4_lo = i4 * kBracketLo;
  c.i4_hi = i4 * kBracketHi;
  c.inv_g = __builtin_amdgcn_rcpf(s_g);
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

// ---- FourOverSix block scaling ----------------------------------------------
//
// Per block, the usual scale byte (block maximum -> 6) or the one that maps the
// block maximum to 4, whichever dequantizes with the smaller sum of squared
// errors (equal errors keep the usual one); a reading of the FourOverSix backend
// the pages name without defining it.

// Exact choice between adjacent scale bytes lo < hi for amax_b / (4 s_g), as
// scale_pick does for 6: midpoint * 4 has <= 6 significant bits.
__device__ __forceinline__ uint32_t scale_pick4(float amax_b, float s_g, uint32_t lo, uint32_t hi) {
  const float mid4 = (e4m3_value(lo) + e4m3_value(hi)) * 2.0f;
  const double d = __builtin_fma(-(double)mid4, (double)s_g, (double)amax_b);
  return d > 0.0 ? hi : (d < 0.0 ? lo : ((lo & 1u) ? hi : lo));
}

__device__ __noinline__ uint32_t scale4_resolve(float amax_b, float s_g, uint32_t c) {
  if (c < 0x7Eu && scale_pick4(amax_b, s_g, c, c + 1) == c + 1) return c + 1;
  if (c > 0u && scale_pick4(amax_b, s_g, c - 1, c) == c - 1) return c - 1;
  return c;
}

// RNE_SAT_E4M3(amax_b / (4 s_g)), bracketed like encode_scale.
__device__ __forceinline__ uint32_t encode_scale4(float amax_b, const EncodeConsts& c) {
  if (c.mode == 1) return 0u;
  if (c.mode == 2) {
    const double r = (double)amax_b / (4.0 * (double)c.s_g);
    return scale4_resolve(amax_b, c.s_g, e4m3_rne_sat((float)r));
  }
  const uint32_t lo = e4m3_rne_sat(amax_b * c.i4_lo);
  const uint32_t hi = e4m3_rne_sat(amax_b * c.i4_hi);
  return lo == hi ? lo : scale_pick4(amax_b, c.s_g, lo, hi);
}

// acc + sum over 8 elements of (x - val(code) sv s_g)^2 in fp64.  val(code) sv
// is exact in fp32 (<= 6 significant bits) and its product with s_g exact in
// fp64; for the values of one block the difference spans well under 53 bits,
// so each d is exact and only the squares and the sum round.
__device__ __forceinline__ double sq_err8(const float (&f)[8], uint32_t w, float sv, double g, double acc) {
  f32x2 v[4];
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const double d0 = __builtin_fma(-(double)(v[j].x * sv), g, (double)f[2 * j]);
    const double d1 = __builtin_fma(-(double)(v[j].y * sv), g, (double)f[2 * j + 1]);
    acc = __builtin_fma(d0, d0, acc);
    acc = __builtin_fma(d1, d1, acc);
  }
  return acc;
}

// Integer significand m and the exponent of its lowest bit, v = m 2^e exactly
// (m odd, or 0 for v == 0), for a finite double.
__device__ __forceinline__ void split_dyadic(double v, int64_t& m, int& e) {
  const uint64_t b = (uint64_t)__builtin_bit_cast(int64_t, v);
  const int be = (int)((b >> 52) & 0x7ff);
  uint64_t mant = b & ((uint64_t(1) << 52) - 1);
  if (be) mant |= uint64_t(1) << 52;
  if (!mant) {
    m = 0;
    e = 0;
    return;
  }
  const int tz = __builtin_ctzll(mant);
  m = (int64_t)(mant >> tz);
  e = (be ? be - 1075 : -1074) + tz;
  if (b >> 63) m = -m;
}

// Exact sign of E4 - E6 for the 16 values of a block, the candidates' values
// y = p s_g (p exact fp32 products, s_g fp32): only elements whose two values
// differ contribute; over them every value is an integer multiple of 2^lo, and
// (x - y4)^2 - (x - y6)^2 = (y6 - y4)(2x - y4 - y6) is summed in 128-bit
// integers (the values of one block span < 40 bits, far inside that).
__device__ __noinline__ int sq_err_sign_exact(const float* x, const float* p4, const float* p6, float s_g) {
  const double g = (double)s_g;
  int lo = 0x7fffffff;
  for (int i = 0; i < 16; i++) {
    const double y4 = (double)p4[i] * g, y6 = (double)p6[i] * g;
    if (y4 == y6) continue;
    const double v[3] = {(double)x[i], y4, y6};
    for (int j = 0; j < 3; j++) {
      int64_t m;
      int e;
      split_dyadic(v[j], m, e);
      if (m && e < lo) lo = e;
    }
  }
  if (lo == 0x7fffffff) return 0;
  __int128 acc = 0;
  for (int i = 0; i < 16; i++) {
    const double y4 = (double)p4[i] * g, y6 = (double)p6[i] * g;
    if (y4 == y6) continue;
    const double v[3] = {(double)x[i], y4, y6};
    __int128 n[3];
    for (int j = 0; j < 3; j++) {
      int64_t m;
      int e;
      split_dyadic(v[j], m, e);
      n[j] = m ? (__int128)m << (e - lo) : (__int128)0;
    }
    acc += (n[2] - n[1]) * (2 * n[0] - n[1] - n[2]);
  }
  return acc > 0 ? 1 : (acc < 0 ? -1 : 0);
}

// Values val(code) sv of the 8 codes of w (exact fp32).
__device__ __forceinline__ void decode8(uint32_t w, float sv, float* p) {
  f32x2 v[4];
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    p[2 * j] = v[j].x * sv;
    p[2 * j + 1] = v[j].y * sv;
  }
}

__device__ __noinline__ bool prefer4_exact(const float (&f0)[8], const float (&f1)[8], uint32_t w6a, uint32_t w6b,
                                           float v6, uint32_t w4a, uint32_t w4b, float v4, float s_g) {
  float x[16], p4[16], p6[16];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    x[i] = f0[i];
    x[8 + i] = f1[i];
  }
  decode8(w4a, v4, p4);
  decode8(w4b, v4, p4 + 8);
  decode8(w6a, v6, p6);
  decode8(w6b, v6, p6 + 8);
  return sq_err_sign_exact(x, p4, p6, s_g) < 0;
}

// The fp64 comparison: the sums carry at most ~2^-48 relative error, so a
// difference beyond 2^-44 of their sum decides; nearer (exact ties included)
// the integer comparison does.
__device__ __noinline__ bool prefer4_f64(const float (&f0)[8], const float (&f1)[8], uint32_t w6a, uint32_t w6b,
                                         float v6, uint32_t w4a, uint32_t w4b, float v4, float s_g) {
  const double g = (double)s_g;
  const double e6 = sq_err8(f1, w6b, v6, g, sq_err8(f0, w6a, v6, g, 0.0));
  if (e6 == 0.0) return false;  // the usual scale is exact: nothing does better
  const double e4 = sq_err8(f1, w4b, v4, g, sq_err8(f0, w4a, v4, g, 0.0));
  const double diff = e6 - e4, tol = 0x1p-44 * (e6 + e4);
  if (diff > tol) return true;
  if (diff < -tol) return false;
  return prefer4_exact(f0, f1, w6a, w6b, v6, w4a, w4b, v4, s_g);
}

// acc + sum over 8 elements of (xs - val(code) sv gn)^2 in fp32, xs = x 2^-g_exp
// and gn = s_g 2^-g_exp (both exact): each difference is one rounding of the
// exact one (fma), each step of the sum one more.
__device__ __forceinline__ float sq_err8_f32(const float* xs, uint32_t w, float sv, float gn, float acc) {
  f32x2 v[4];
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float d0 = __builtin_fmaf(-(v[j].x * sv), gn, xs[2 * j]);
    const float d1 = __builtin_fmaf(-(v[j].y * sv), gn, xs[2 * j + 1]);
    acc = __builtin_fmaf(d0, d0, acc);
    acc = __builtin_fmaf(d1, d1, acc);
  }
  return acc;
}

// Whether the block (f0, f1) encoded under scale byte sb4 (codes w4a, w4b)
// has a smaller squared error than under the usual sb6 (codes w6a, w6b), in
// fp32 on the block scaled by 2^-g_exp (exact; a block whose two candidates
// differ lies below ~2600 s_g, so nothing overflows): each sum is within
// 18 2^-24 of its exact value, so a difference beyond 2^-16 of their sum
// decides, provided the sums are far from the fp32 subnormal range.  Returns
// 1 (sb4), 0 (sb6) or -1: undecided (near-ties, exact ties, sums of zero),
// for prefer4_f64 to settle.  No calls: it sits in the encode loops.
__device__ __forceinline__ int prefer4_fast(const float (&f0)[8], const float (&f1)[8], uint32_t w6a, uint32_t w6b,
                                            uint32_t sb6, uint32_t w4a, uint32_t w4b, uint32_t sb4,
                                            const EncodeConsts& c) {
  const float v6 = e4m3_value(sb6), v4 = e4m3_value(sb4);
  float xs[16];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    xs[i] = __builtin_ldexpf(f0[i], -c.g_exp);
    xs[8 + i] = __builtin_ldexpf(f1[i], -c.g_exp);
  }
  const float e6 = sq_err8_f32(xs + 8, w6b, v6, c.g_norm, sq_err8_f32(xs, w6a, v6, c.g_norm, 0.0f));
  const float e4 = sq_err8_f32(xs + 8, w4b, v4, c.g_norm, sq_err8_f32(xs, w4a, v4, c.g_norm, 0.0f));
  const float sum = e6 + e4, diff = e6 - e4, tol = 0x1p-16f * sum;
  if (__builtin_expect(sum >= 0x1p-100f, 1)) {
    if (diff > tol) return 1;
    if (diff < -tol) return 0;
  }
  return -1;
}

// The same decision, always settled (prefer4_fast, then the fp64 and exact
// comparisons).
__device__ __forceinline__ bool prefer4(const float (&f0)[8], const float (&f1)[8], uint32_t w6a, uint32_t w6b,
                                        uint32_t sb6, uint32_t w4a, uint32_t w4b, uint32_t sb4, const EncodeConsts& c) {
  const int d = prefer4_fast(f0, f1, w6a, w6b, sb6, w4a, w4b, sb4, c);
  if (d >= 0) return d == 1;
  return prefer4_f64(f0, f1, w6a, w6b, e4m3_value(sb6), w4a, w4b, e4m3_value(sb4), c.s_g);
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
