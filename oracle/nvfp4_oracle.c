/*
 * NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, exact reference for what the GPU library computes.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it; the product path never does.  It shares no code, header or table
 * with the HIP library.
 *
 * What it follows.  The pages (LongLive-2.0: "An NVFP4 Parallel Infrastructure
 * for Long Video Generation", arXiv abstract page, Abstract; d9249.github.io
 * review, section "Core idea / structure / operation") say the DiT linears run
 * W4A4 NVFP4 and that the KV cache is stored as NVFP4 and restored by a
 * dequantization kernel, but they define no numeric detail.  The numeric
 * contract used here is:
 *   - E2M1 element codes on the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (with sign),
 *     OCP Microscaling v1.0 bit layout: bit 3 sign, bits 2:1 exponent (bias 1),
 *     bit 0 mantissa; element 2i in the low nibble of byte i.
 *   - one E4M3 scale byte (OCP FP8 E4M3FN: bias 7, max 448 = 0x7E, 0x7F NaN)
 *     per 16 contiguous elements along the reduction axis;
 *   - one fp32 per-tensor (per-head for the KV cache) scale
 *     s_g = RN_f32(amax / (6 * 448));
 *   - block scale s_b = RNE_SAT_E4M3(amax_block / (6 * s_g));
 *   - code q = RNE_SAT_E2M1(x / (val(s_b) * s_g)), sign always kept;
 *   - dequantized value = RN_out(val(q) * val(s_b) * s_g).
 * Every rounding is ONE round-to-nearest-even of the exact real value, with
 * ties going to the even code / even byte / even significand.  Every decision
 * below is taken by comparing the input with an exactly representable
 * boundary (a midpoint times the scale, exact in fp64), so no division
 * rounding enters any decision.
 *
 * All entry points return 0 on success and a negative value on a non-finite
 * input or a bad shape.  Arrays are host memory, row-major, reduction axis
 * contiguous.  OpenMP runs over rows.
 */
#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* exact fp64 values (results of the oracle's own fp64 arithmetic) */
#define ORC_OK 0
#define ORC_ERR_NONFINITE (-1)
#define ORC_ERR_SHAPE (-2)

int orc_version(void) { return 1; }

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the OpenMP loops that follow (timing on one core or on all);
 * the results do not depend on it. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---- scalar formats -------------------------------------------------- */

/* bf16 bit pattern -> its exact value. */
static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double load_elem(const void *x, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float *)x)[i];
  if (dtype == ORC_F64) return ((const double *)x)[i];
  return bf16_to_double(((const uint16_t *)x)[i]);
}

/* E2M1 nibble -> value.  Magnitude 2^(e-1) * (1 + m/2) for e >= 1 and
 * m/2 for e == 0; bit 3 is the sign (0x8 is -0.0). */
double orc_e2m1_value(int code) {
  int e = (code >> 1) & 3, m = code & 1;
  double mag = e ? ldexp(1.0 + m / 2.0, e - 1) : m / 2.0;
  return (code & 8) ? -mag : mag;
}

/* E4M3FN byte -> value.  2^(e-7) * (1 + m/8) for e >= 1, 2^-6 * m/8 for
 * e == 0; exponent 15 with mantissa 7 is NaN (no infinities). */
double orc_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return s ? -mag : mag;
}

/* s_g = RN_f32(amax / 2688): the float nearest to the exact quotient, ties to
 * the even significand.  The fp64 quotient gives a candidate within one fp32
 * ulp; the exact choice is made among it and its two neighbours by comparing
 * |f * 2688 - amax|, which is exact in fp64 (f*2688 has at most 29
 * significant bits and the two terms are within a factor of two). */
float orc_global_scale_f64(double amax);
float orc_global_scale(float amax) { return orc_global_scale_f64((double)amax); }

/* The same rounding for an fp64 amax: f * 2688 is exact (<= 36 bits) and
 * within a factor of two of amax, so the difference is exact as well. */
float orc_global_scale_f64(double amax) {
  if (!(amax > 0.0)) return 0.0f;
  float c = (float)(amax / 2688.0);
  float cand[3] = {nextafterf(c, 0.0f), c, nextafterf(c, INFINITY)};
  float best = cand[0];
  double best_err = INFINITY;
  for (int i = 0; i < 3; i++) {
    double err = fabs((double)cand[i] * 2688.0 - amax);
    uint32_t bits;
    memcpy(&bits, &cand[i], 4);
    if (err < best_err || (err == best_err && (bits & 1u) == 0)) {
      best = cand[i];
      best_err = err;
    }
  }
  return best;
}

/* Block scale byte: RNE_SAT_E4M3(amax_b / (6 s_g)).  The ratio is placed
 * among the 127 finite non-negative E4M3 values by comparing amax_b with
 * midpoint(b-1, b) * 6 * s_g, exact in fp64 (<= 5 + 2 + 24 significant
 * bits).  At a midpoint the even byte wins; anything above the last
 * midpoint (432) saturates to 0x7E = 448; a zero s_g or zero block gives 0. */
static int block_scale_div(double amax_b, float s_g, double div) {
  if (s_g == 0.0f || amax_b == 0.0) return 0;
  double den = div * (double)s_g;
  int best = 0;
  for (int b = 1; b < 127; b++) {
    double mid = 0.5 * (orc_e4m3_value(b - 1) + orc_e4m3_value(b)) * den;
    if (amax_b > mid || (amax_b == mid && (b % 2) == 0)) best = b;
  }
  return best;
}

int orc_block_scale(double amax_b, float s_g) { return block_scale_div(amax_b, s_g, 6.0); }

/* The same rounding of amax_b / (4 s_g): the scale that maps the block maximum
 * to 4 instead of 6 (the second candidate of FourOverSix below); mid * 4 * s_g
 * is exact in fp64 as well. */
int orc_block_scale4(double amax_b, float s_g) { return block_scale_div(amax_b, s_g, 4.0); }

/* Element code: sign(x) | RNE_SAT_E2M1(|x| / S) with S = val(s_b) * s_g
 * (exact in fp64).  |x| is compared with midpoint(i-1, i) * S, exact in
 * fp64 (<= 3 + 4 + 24 significant bits); ties take the even code; above
 * 5 S everything saturates to 6 (code 7).  S == 0 keeps only the sign. */
int orc_e2m1_code(double x, double S) {
  int sign = signbit(x) ? 8 : 0;
  if (S == 0.0) return sign;
  double a = fabs(x);
  int best = 0;
  for (int i = 1; i < 8; i++) {
    double mid = 0.5 * (orc_e2m1_value(i - 1) + orc_e2m1_value(i)) * S;
    if (a > mid || (a == mid && (i % 2) == 0)) best = i;
  }
  return sign | best;
}

/* One round-to-nearest-even of an exact fp64 value to bfloat16 (8
 * significant bits, fp32 exponent range, subnormal step 2^-133).  Returns the
 * bf16 bit pattern. */
uint16_t orc_round_bf16(double v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  uint16_t sign = neg ? 0x8000 : 0;
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E); /* a = f * 2^E, f in [0.5, 1): leading bit has weight 2^(E-1) */
  int ulp_exp = E - 8;
  if (ulp_exp < -133) ulp_exp = -133;
  double q = ldexp(a, -ulp_exp); /* exact: power-of-two scaling */
  double qf = floor(q);
  double frac = q - qf;
  if (frac > 0.5 || (frac == 0.5 && fmod(qf, 2.0) != 0.0)) qf += 1.0;
  double r = ldexp(qf, ulp_exp);
  if (r >= ldexp(1.0, 128)) return sign | 0x7f80; /* overflow to infinity */
  float rf = (float)r; /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &rf, 4);
  return sign | (uint16_t)((u >> 16) & 0x7fff);
}

/* ---- tensors --------------------------------------------------------- */

/* amax = max |x| over n elements (exact). */
int orc_amax(const void *x, int dtype, int64_t n, float *amax) {
  if (dtype == ORC_F64) return ORC_ERR_SHAPE; /* the maximum of fp64 values need not be an fp32 value */
  double m = 0.0;
  for (int64_t i = 0; i < n; i++) {
    double v = load_elem(x, dtype, i);
    if (!isfinite(v)) return ORC_ERR_NONFINITE;
    if (fabs(v) > m) m = fabs(v);
  }
  *amax = (float)m; /* exact: m is an input value */
  return ORC_OK;
}

/* Quantize rows x k elements with a given s_g into codes [rows][k/2] and
 * scale bytes [rows][k/16]. */
int orc_quantize_with_scale(const void *x, int dtype, int64_t rows, int64_t k, float s_g,
                            uint8_t *codes, uint8_t *scales) {
  if (rows < 0 || k <= 0 || k % 16 != 0) return ORC_ERR_SHAPE;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t blk = 0; blk < k / 16; blk++) {
      double v[16];
      double amax_b = 0.0;
      for (int i = 0; i < 16; i++) {
        v[i] = load_elem(x, dtype, r * k + blk * 16 + i);
        if (!isfinite(v[i])) bad = 1;
        if (fabs(v[i]) > amax_b) amax_b = fabs(v[i]);
      }
      int sb = orc_block_scale(amax_b, s_g);
      double S = orc_e4m3_value(sb) * (double)s_g; /* exact */
      scales[r * (k / 16) + blk] = (uint8_t)sb;
      for (int i = 0; i < 16; i += 2) {
        int lo = orc_e2m1_code(v[i], S), hi = orc_e2m1_code(v[i + 1], S);
        codes[r * (k / 2) + blk * 8 + i / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
  return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* Full per-tensor quantization: amax -> s_g -> blocks.  For fp64 inputs the
 * amax is an fp64 value and s_g its exact rounding. */
int orc_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                 uint8_t *scales, float *s_g) {
  if (rows < 0 || k <= 0 || k % 16 != 0) return ORC_ERR_SHAPE;
  double m = 0.0;
  for (int64_t i = 0; i < rows * k; i++) {
    double v = load_elem(x, dtype, i);
    if (!isfinite(v)) return ORC_ERR_NONFINITE;
    if (fabs(v) > m) m = fabs(v);
  }
  *s_g = orc_global_scale_f64(m);
  return orc_quantize_with_scale(x, dtype, rows, k, *s_g, codes, scales);
}

/* ---- FourOverSix block scaling ---------------------------------------- */

/* The pages name a FourOverSix backend (a `fouroversix` directory) and an
 * NVFP4 checkpoint `model_4o6.pt` (d9249.github.io review, sections on the
 * evidence and on the practical reading) but do not define it.  Reading used
 * here (not fixed by the pages): s_g is the usual per-tensor scale; for each
 * 16-element block two candidate scale bytes are formed, s6 = RNE_SAT(amax_b /
 * (6 s_g)) (the standard one) and s4 = RNE_SAT(amax_b / (4 s_g)), the block is
 * encoded under each with the usual E2M1 rounding, and the candidate whose
 * dequantized block val(q) val(s) s_g has the smaller sum of squared errors
 * against the input is kept; equal errors keep s6.  The stored format is plain
 * NVFP4, so dequantization and the GEMM are unchanged. */

/* Exponent of the lowest and of the highest set bit of a finite nonzero double. */
static int low_bit_exp(double v) {
  int e;
  double m = frexp(fabs(v), &e); /* |v| = m 2^e, m in [0.5, 1) */
  uint64_t u = (uint64_t)ldexp(m, 53);
  return e - 53 + __builtin_ctzll(u);
}

static int high_bit_exp(double v) {
  int e;
  frexp(fabs(v), &e);
  return e - 1;
}

/* Sign of sum_i (x_i - a_i)^2 - sum_i (x_i - b_i)^2, exactly, for exact double
 * values.  Elements with a_i == b_i contribute nothing; for the others every
 * nonzero value is an integer multiple of 2^lo (lo the lowest set bit among
 * them), and (x - a)^2 - (x - b)^2 = (b - a)(2x - a - b) is summed in 128-bit
 * integers.  Returns -2 if the values span more than 56 bits (then the sum
 * could overflow; it cannot happen for the values of one block). */
static int cmp_sq_err(const double *x, const double *a, const double *b, int n) {
  int lo = INT_MAX, hi = INT_MIN;
  for (int i = 0; i < n; i++) {
    if (a[i] == b[i]) continue;
    const double v[3] = {x[i], a[i], b[i]};
    for (int j = 0; j < 3; j++)
      if (v[j] != 0.0) {
        if (low_bit_exp(v[j]) < lo) lo = low_bit_exp(v[j]);
        if (high_bit_exp(v[j]) > hi) hi = high_bit_exp(v[j]);
      }
  }
  if (lo == INT_MAX) return 0;
  if (hi - lo > 56) return -2;
  __int128 d = 0;
  for (int i = 0; i < n; i++) {
    if (a[i] == b[i]) continue;
    const __int128 X = (__int128)(int64_t)ldexp(x[i], -lo), A = (__int128)(int64_t)ldexp(a[i], -lo),
                   B = (__int128)(int64_t)ldexp(b[i], -lo);
    d += (B - A) * (2 * X - A - B);
  }
  return d > 0 ? 1 : (d < 0 ? -1 : 0);
}

/* FourOverSix quantization of rows x k elements with a given s_g. */
int orc_quantize_4o6_with_scale(const void *x, int dtype, int64_t rows, int64_t k, float s_g,
                                uint8_t *codes, uint8_t *scales) {
  if (rows < 0 || k <= 0 || k % 16 != 0) return ORC_ERR_SHAPE;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t blk = 0; blk < k / 16; blk++) {
      double v[16], y6[16], y4[16];
      int c6[16], c4[16];
      double amax_b = 0.0;
      for (int i = 0; i < 16; i++) {
        v[i] = load_elem(x, dtype, r * k + blk * 16 + i);
        if (!isfinite(v[i])) bad = 1;
        if (fabs(v[i]) > amax_b) amax_b = fabs(v[i]);
      }
      const int s6 = orc_block_scale(amax_b, s_g), s4 = orc_block_scale4(amax_b, s_g);
      const double S6 = orc_e4m3_value(s6) * (double)s_g, S4 = orc_e4m3_value(s4) * (double)s_g; /* exact */
      for (int i = 0; i < 16; i++) {
        c6[i] = orc_e2m1_code(v[i], S6);
        c4[i] = orc_e2m1_code(v[i], S4);
        y6[i] = orc_e2m1_value(c6[i]) * S6; /* exact: <= 2 + 4 + 24 significant bits */
        y4[i] = orc_e2m1_value(c4[i]) * S4;
      }
      int use4 = 0;
      if (s4 != s6) {
        const int c = cmp_sq_err(v, y4, y6, 16); /* sign of E(s4) - E(s6) */
        if (c == -2) bad = 2;
        use4 = (c == -1);
      }
      const int *cc = use4 ? c4 : c6;
      scales[r * (k / 16) + blk] = (uint8_t)(use4 ? s4 : s6);
      for (int i = 0; i < 16; i += 2)
        codes[r * (k / 2) + blk * 8 + i / 2] = (uint8_t)(cc[i] | (cc[i + 1] << 4));
    }
  }
  return bad == 1 ? ORC_ERR_NONFINITE : (bad ? ORC_ERR_SHAPE : ORC_OK);
}

/* FourOverSix with the per-tensor scale computed as usual (amax / 2688). */
int orc_quantize_4o6(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes, uint8_t *scales,
                     float *s_g) {
  if (rows < 0 || k <= 0 || k % 16 != 0) return ORC_ERR_SHAPE;
  double m = 0.0;
  for (int64_t i = 0; i < rows * k; i++) {
    double v = load_elem(x, dtype, i);
    if (!isfinite(v)) return ORC_ERR_NONFINITE;
    if (fabs(v) > m) m = fabs(v);
  }
  *s_g = orc_global_scale_f64(m);
  return orc_quantize_4o6_with_scale(x, dtype, rows, k, *s_g, codes, scales);
}

/* adaLN of layer-normalized rows (the pages list a unified RoPE + adaLN kernel
 * among the NVFP4 inference-path optimizations: yourai.pro news page), in
 * fp64.  For row r of x [rows][k] and its group g = r / rows_per_group:
 *   mu  = sum_d x[r][d] / k,   var = sum_d (x[r][d] - mu)^2 / k  (biased),
 *   y[r][d] = (x[r][d] - mu) / sqrt(var + eps) * (1 + scale[g][d]) + shift[g][d],
 * shift and scale fp32 [groups][k].  The result feeds orc_quantize as fp64. */
int orc_adaln(const void *x, int dtype, int64_t rows, int64_t k, const float *shift, const float *scale,
              int64_t rows_per_group, double eps, double *y) {
  if (rows < 0 || k <= 0 || rows_per_group <= 0 || !(eps >= 0.0)) return ORC_ERR_SHAPE;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    const int64_t g = r / rows_per_group;
    double mu = 0.0, var = 0.0;
    for (int64_t d = 0; d < k; d++) mu += load_elem(x, dtype, r * k + d);
    mu /= (double)k;
    for (int64_t d = 0; d < k; d++) {
      double c = load_elem(x, dtype, r * k + d) - mu;
      var += c * c;
    }
    var /= (double)k;
    if (!isfinite(mu) || !isfinite(var)) bad = 1;
    const double rstd = 1.0 / sqrt(var + eps);
    for (int64_t d = 0; d < k; d++) {
      const double c = load_elem(x, dtype, r * k + d) - mu;
      y[r * k + d] = c * rstd * (1.0 + (double)scale[g * k + d]) + (double)shift[g * k + d];
      if (!isfinite(y[r * k + d])) bad = 1;
    }
  }
  return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* y = RN_out(val(q) * val(s_b) * s_g); the product is exact in fp64
 * (<= 2 + 4 + 24 significant bits) and rounded once. */
int orc_dequantize(const uint8_t *codes, const uint8_t *scales, float s_g, int64_t rows, int64_t k,
                   void *y, int y_dtype) {
  if (rows < 0 || k <= 0 || k % 16 != 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t i = 0; i < k; i++) {
      int byte = codes[r * (k / 2) + i / 2];
      int q = (i & 1) ? (byte >> 4) : (byte & 15);
      double v = orc_e2m1_value(q) * orc_e4m3_value(scales[r * (k / 16) + i / 16]) * (double)s_g;
      if (y_dtype == ORC_F32)
        ((float *)y)[r * k + i] = (float)v; /* one RNE of the exact value */
      else
        ((uint16_t *)y)[r * k + i] = orc_round_bf16(v);
    }
  }
  return ORC_OK;
}

/* Exact decoded row without s_g: d[i] = val(q_i) * val(s_b(i)) (<= 6 bits). */
static void decode_row(const uint8_t *codes, const uint8_t *scales, int64_t k, int64_t r, double *d) {
  for (int64_t i = 0; i < k; i++) {
    int byte = codes[r * (k / 2) + i / 2];
    int q = (i & 1) ? (byte >> 4) : (byte & 15);
    d[i] = orc_e2m1_value(q) * orc_e4m3_value(scales[r * (k / 16) + i / 16]);
  }
}

/* GEMM reference for C = A . B^T with A [M][K], B [N][K] in NVFP4:
 *   ref[i][j] = s_gA s_gB sum_k a_k b_k,  abssum[i][j] = s_gA s_gB sum_k |a_k b_k|
 * over the selected rows (row_idx, n_rows; NULL = all M) and columns (col_idx,
 * n_cols; NULL = all N).  Each a_k b_k is exact in fp64 (<= 12 bits); the sum
 * runs in fp64 in k order, the relative error is below K * 2^-53. */
int orc_gemm_ref(const uint8_t *a_codes, const uint8_t *a_scales, float a_sg, const uint8_t *b_codes,
                 const uint8_t *b_scales, float b_sg, int64_t M, int64_t N, int64_t K,
                 const int64_t *row_idx, int64_t n_rows, const int64_t *col_idx, int64_t n_cols,
                 double *ref, double *abssum) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return ORC_ERR_SHAPE;
  int64_t nr = row_idx ? n_rows : M, nc = col_idx ? n_cols : N;
  for (int64_t i = 0; i < nr; i++)
    if (row_idx && (row_idx[i] < 0 || row_idx[i] >= M)) return ORC_ERR_SHAPE;
  for (int64_t j = 0; j < nc; j++)
    if (col_idx && (col_idx[j] < 0 || col_idx[j] >= N)) return ORC_ERR_SHAPE;
  double gscale = (double)a_sg * (double)b_sg; /* exact: 24 x 24 bits */
  /* Decode the selected B rows once; each A row is decoded by its thread. */
  double *bd = (double *)malloc(sizeof(double) * (size_t)(nc * K));
  if (!bd) return ORC_ERR_SHAPE;
  for (int64_t j = 0; j < nc; j++) decode_row(b_codes, b_scales, K, col_idx ? col_idx[j] : j, bd + j * K);
  int fail = 0;
#pragma omp parallel reduction(| : fail)
  {
    double *ad = (double *)malloc(sizeof(double) * (size_t)K);
    if (!ad) fail = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nr; i++) {
      if (!ad) continue;
      decode_row(a_codes, a_scales, K, row_idx ? row_idx[i] : i, ad);
      for (int64_t j = 0; j < nc; j++) {
        const double *b = bd + j * K;
        double s = 0.0, t = 0.0;
        for (int64_t kk = 0; kk < K; kk++) {
          double p = ad[kk] * b[kk];
          s += p;
          t += fabs(p);
        }
        ref[i * nc + j] = s * gscale;
        abssum[i * nc + j] = t * gscale;
      }
    }
    free(ad);
  }
  free(bd);
  return fail ? ORC_ERR_SHAPE : ORC_OK;
}

/* ---- NVFP4 KV cache: [heads][tokens][head_dim], one s_g per head ------ */

/* Per head h: s_g[h] = RN_f32(amax over the head's tokens x head_dim / 2688),
 * then the same 16-element blocks along head_dim as above. */
int orc_kv_quantize(const uint16_t *kv, int64_t heads, int64_t tokens, int64_t head_dim,
                    uint8_t *codes, uint8_t *scales, float *head_scales) {
  if (heads <= 0 || tokens < 0 || head_dim <= 0 || head_dim % 16 != 0) return ORC_ERR_SHAPE;
  for (int64_t h = 0; h < heads; h++) {
    const uint16_t *xh = kv + h * tokens * head_dim;
    float amax;
    int st = orc_amax(xh, ORC_BF16, tokens * head_dim, &amax);
    if (st) return st;
    head_scales[h] = orc_global_scale(amax);
    st = orc_quantize_with_scale(xh, ORC_BF16, tokens, head_dim, head_scales[h],
                                 codes + h * tokens * (head_dim / 2),
                                 scales + h * tokens * (head_dim / 16));
    if (st) return st;
  }
  return ORC_OK;
}

/* The same per-head scales with FourOverSix block scaling (see above). */
int orc_kv_quantize_4o6(const uint16_t *kv, int64_t heads, int64_t tokens, int64_t head_dim,
                        uint8_t *codes, uint8_t *scales, float *head_scales) {
  if (heads <= 0 || tokens < 0 || head_dim <= 0 || head_dim % 16 != 0) return ORC_ERR_SHAPE;
  for (int64_t h = 0; h < heads; h++) {
    const uint16_t *xh = kv + h * tokens * head_dim;
    float amax;
    int st = orc_amax(xh, ORC_BF16, tokens * head_dim, &amax);
    if (st) return st;
    head_scales[h] = orc_global_scale(amax);
    st = orc_quantize_4o6_with_scale(xh, ORC_BF16, tokens, head_dim, head_scales[h],
                                     codes + h * tokens * (head_dim / 2),
                                     scales + h * tokens * (head_dim / 16));
    if (st) return st;
  }
  return ORC_OK;
}

/* Per head: bf16 = RN_bf16(val(q) * val(s_b) * s_g[h]). */
int orc_kv_dequantize(const uint8_t *codes, const uint8_t *scales, const float *head_scales,
                      int64_t heads, int64_t tokens, int64_t head_dim, uint16_t *out) {
  if (heads <= 0 || tokens < 0 || head_dim <= 0 || head_dim % 16 != 0) return ORC_ERR_SHAPE;
  for (int64_t h = 0; h < heads; h++) {
    int st = orc_dequantize(codes + h * tokens * (head_dim / 2), scales + h * tokens * (head_dim / 16),
                            head_scales[h], tokens, head_dim, out + h * tokens * head_dim, ORC_BF16);
    if (st) return st;
  }
  return ORC_OK;
}

/* ---- attention over an NVFP4 KV cache ---------------------------------- */

/* Exact dequantized cache row (val(q) val(s_b) s_g, <= 30 significant bits:
 * exact in fp64). */
static void decode_kv_row(const uint8_t *codes, const uint8_t *scales, float s_g, int64_t d, int64_t row,
                          double *out) {
  decode_row(codes, scales, d, row, out);
  for (int64_t i = 0; i < d; i++) out[i] *= (double)s_g;
}

/* Softmax attention of bf16 queries over the first kv_tokens rows of an NVFP4
 * K/V cache (the pages: the NVFP4 KV cache is restored by a parallel
 * dequantization kernel and read by the attention).  For head h, query i:
 *   s_j = scale * sum_d q[i][d] k[j][d],  w_j = exp(s_j - max_j s_j),
 *   out[i][d]  = sum_j w_j v[j][d] / sum_j w_j,
 *   wabs[i][d] = sum_j w_j |v[j][d]| / sum_j w_j,
 *   lsum[i]    = sum_j w_j  (the softmax normaliser, >= 1),
 * with k, v the exact dequantized rows; fp64 throughout, token order.  The
 * cache is [heads][cache_tokens][...]; q and the outputs [heads][q_tokens or
 * n_q][head_dim] (lsum [heads][q_tokens or n_q], optional: NULL skips it).
 * q_idx (n_q entries) restricts the queries of every head; NULL computes all
 * q_tokens. */
int orc_kv_attention(const uint16_t *q, int64_t heads, int64_t q_tokens, int64_t head_dim,
                     const uint8_t *k_codes, const uint8_t *k_scales, const float *k_hs,
                     const uint8_t *v_codes, const uint8_t *v_scales, const float *v_hs,
                     int64_t cache_tokens, int64_t kv_tokens, double scale, const int64_t *q_idx,
                     int64_t n_q, double *out, double *wabs, double *lsum) {
  if (heads <= 0 || q_tokens < 0 || head_dim <= 0 || head_dim % 16 != 0 || kv_tokens <= 0 ||
      kv_tokens > cache_tokens || !isfinite(scale))
    return ORC_ERR_SHAPE;
  const int64_t nq = q_idx ? n_q : q_tokens;
  for (int64_t i = 0; i < nq; i++)
    if (q_idx && (q_idx[i] < 0 || q_idx[i] >= q_tokens)) return ORC_ERR_SHAPE;
  const int64_t D = head_dim, T = kv_tokens;
  double *kd = (double *)malloc(sizeof(double) * (size_t)(T * D));
  double *vd = (double *)malloc(sizeof(double) * (size_t)(T * D));
  if (!kd || !vd) {
    free(kd);
    free(vd);
    return ORC_ERR_SHAPE;
  }
  int fail = 0;
  for (int64_t h = 0; h < heads && !fail; h++) {
    const uint8_t *kc = k_codes + h * cache_tokens * (D / 2), *ks = k_scales + h * cache_tokens * (D / 16);
    const uint8_t *vc = v_codes + h * cache_tokens * (D / 2), *vs = v_scales + h * cache_tokens * (D / 16);
    for (int64_t j = 0; j < T; j++) {
      decode_kv_row(kc, ks, k_hs[h], D, j, kd + j * D);
      decode_kv_row(vc, vs, v_hs[h], D, j, vd + j * D);
    }
#pragma omp parallel reduction(| : fail)
    {
      double *s = (double *)malloc(sizeof(double) * (size_t)T);
      double *qd = (double *)malloc(sizeof(double) * (size_t)D);
      if (!s || !qd) fail = 1;
#pragma omp for schedule(dynamic, 1)
      for (int64_t ii = 0; ii < nq; ii++) {
        if (!s || !qd) continue;
        const int64_t i = q_idx ? q_idx[ii] : ii;
        for (int64_t d = 0; d < D; d++) {
          qd[d] = bf16_to_double(q[(h * q_tokens + i) * D + d]);
          if (!isfinite(qd[d])) fail = 1;
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < T; j++) {
          double dot = 0.0;
          for (int64_t d = 0; d < D; d++) dot += qd[d] * kd[j * D + d];
          s[j] = scale * dot;
          if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < T; j++) {
          s[j] = exp(s[j] - m);
          l += s[j];
        }
        double *o = out + (h * nq + ii) * D, *wa = wabs + (h * nq + ii) * D;
        for (int64_t d = 0; d < D; d++) o[d] = wa[d] = 0.0;
        for (int64_t j = 0; j < T; j++)
          for (int64_t d = 0; d < D; d++) {
            o[d] += s[j] * vd[j * D + d];
            wa[d] += s[j] * fabs(vd[j * D + d]);
          }
        for (int64_t d = 0; d < D; d++) {
          o[d] /= l;
          wa[d] /= l;
        }
        if (lsum) lsum[h * nq + ii] = l;
      }
      free(s);
      free(qd);
    }
  }
  free(kd);
  free(vd);
  return fail ? ORC_ERR_NONFINITE : ORC_OK;
}
