/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 library: block quantization,
 * dequantization, the W4A4 block-scaled GEMM of the DiT linears and the
 * NVFP4 KV cache.
 *
 * Where the operations come from.  LongLive-2.0 ("An NVFP4 Parallel
 * Infrastructure for Long Video Generation"): the arXiv abstract page
 * (fugumt.com, Abstract) states that inference on Blackwell runs W4A4 NVFP4
 * and that the KV cache is quantized into NVFP4 to save memory; the
 * d9249.github.io review (section "Core idea / structure / operation") adds
 * that a parallel dequantization kernel restores the NVFP4 KV cache; the
 * yourai.pro news page lists faster FP4 dequantization and reduced KV-cache
 * synchronization among the NVFP4 inference-path optimizations.  The pages
 * fix no numeric detail; the format below is the NVFP4 layout (E2M1 element
 * codes, one E4M3 scale per 16 elements, one fp32 per-tensor scale) with
 * OCP Microscaling v1.0 / OCP FP8 E4M3FN bit encodings.
 *
 * Format (one tensor of `rows` x `k`, k contiguous, k % 16 == 0):
 *   s_g            fp32, = RN_f32(amax / (6 * 448)), amax = max |x| over the
 *                  tensor (over each head for the KV cache);
 *   scales[r][j]   u8 E4M3FN, = RNE_SAT(amax of elements 16j..16j+15 of row r
 *                  / (6 * s_g)); 0 for an all-zero block or s_g == 0;
 *   codes[r][i]    u8, two E2M1 codes: element 2i in bits 3:0, element 2i+1
 *                  in bits 7:4; code = sign bit (bit 3) | RNE_SAT(|x| /
 *                  (val(scale) * s_g)) on {0, .5, 1, 1.5, 2, 3, 4, 6};
 *   dequantized    RN_out(val(code) * val(scale) * s_g), one rounding.
 * Every rounding is one round-to-nearest-even of the exact real value (ties
 * to the even code / byte / significand); results are bit-exact and
 * independent of launch configuration.
 *
 * Conventions for every call:
 *   - pointers are device pointers (HBM) owned by the caller; the library
 *     allocates nothing and keeps no state between calls;
 *   - `stream` is a hipStream_t passed as void* (NULL = null stream); every
 *     call only enqueues work on it and never synchronizes the host;
 *   - arguments are validated before anything is enqueued: on any error
 *     status nothing was launched and no output was touched;
 *   - NVFP4_ERR_LAUNCH reports a failed kernel launch (for example no GPU);
 *     device faults surface at the caller's next synchronization;
 *   - inputs must be finite; NaN/Inf inputs give unspecified outputs;
 *   - data pointers must be 16-byte aligned, scale/s_g pointers 4-byte
 *     aligned (NVFP4_ERR_ALIGN otherwise);
 *   - calls on one stream are ordered; calls on different streams that
 *     share an output buffer race.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 2

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,   /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,  /* a size is negative, zero where not allowed, not a multiple of 16 along k, or too large */
  NVFP4_ERR_ALIGN = 3,  /* a pointer is not aligned as required */
  NVFP4_ERR_DTYPE = 4,  /* unknown dtype */
  NVFP4_ERR_LAUNCH = 5, /* the HIP runtime rejected a launch */
  NVFP4_ERR_FLAGS = 6   /* unknown flags value */
} nvfp4_status_t;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype_t;

/* Size of the fixed device array that kv_attention_noalloc uses as scratch. */
#define NVFP4_NOALLOC_SCRATCH_BYTES (32u << 20)

#define NVFP4_SCALE_COMPUTE 0 /* compute s_g from the data and write it to *s_g */
#define NVFP4_SCALE_GIVEN 1   /* use the s_g already stored at *s_g (device) */
/*
 * FourOverSix block scaling, OR-ed into the flags of the calls that list it.
 * The pages name a FourOverSix backend (a `fouroversix` directory) and an NVFP4
 * checkpoint `model_4o6.pt` (d9249.github.io review, sections on the evidence
 * and on the practical reading) without defining it; the rule here is a
 * reading: s_g as usual; per 16-element block the scale byte is either the
 * usual s6 = RNE_SAT(amax_b / (6 s_g)) or s4 = RNE_SAT(amax_b / (4 s_g)),
 * whichever gives the dequantized block val(q) val(s) s_g the smaller exact
 * sum of squared errors against the input (equal errors: s6), with the codes
 * rounded as usual under the kept scale.  The output is ordinary NVFP4:
 * dequantize, GEMM and attention read it unchanged.
 */
#define NVFP4_FOUR_OVER_SIX 2

/* Version of this ABI (NVFP4_ABI_VERSION). */
int nvfp4_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *nvfp4_status_string(nvfp4_status_t status);

/*
 * Per-tensor scale alone: s_g[0] = RN_f32(max |x| / (6 * 448)) for x
 * [rows][k] (dtype F32 or BF16, row-major), the value nvfp4_quantize
 * computes with NVFP4_SCALE_COMPUTE.  Pass it back with NVFP4_SCALE_GIVEN
 * to quantize several tensors, or chunks of one tensor written at different
 * times, against one scale.  The scale stays on the device (the yourai.pro
 * page lists reduced KV-cache synchronization among the NVFP4 inference-path
 * optimizations: no host round trip).  s_g is also the reduction slot: the
 * call zeroes it, every workgroup folds in its maximum with one atomic max
 * on the magnitude bits (order-free, so deterministic), and a last kernel
 * rounds it in place; s_g must not be read or written by other work until
 * the call has finished on `stream`.  rows == 0 gives s_g = 0.  Requires
 * k > 0, k % 16 == 0, rows * k < 2^40.
 */
nvfp4_status_t nvfp4_global_scale(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t k, float *s_g,
                                  void *stream);

/*
 * Quantize x [rows][k] (dtype F32 or BF16, row-major) to NVFP4.
 *   codes   [rows][k/2]  u8 out      scales [rows][k/16] u8 out
 *   s_g     [1] fp32: out with NVFP4_SCALE_COMPUTE, in with NVFP4_SCALE_GIVEN
 *   flags   NVFP4_SCALE_COMPUTE or NVFP4_SCALE_GIVEN, optionally
 *           | NVFP4_FOUR_OVER_SIX
 * Per the arXiv abstract (W4A4 NVFP4 inference: weights and activations
 * quantized).  rows == 0 is allowed (COMPUTE then writes s_g = 0).  With
 * COMPUTE the call runs three kernels (amax partials, s_g finalize, encode);
 * the codes buffer serves as scratch for the amax partials before it is
 * overwritten.  Requires k > 0, k % 16 == 0, rows * k < 2^40.
 */
nvfp4_status_t nvfp4_quantize(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t k, uint8_t *codes,
                              uint8_t *scales, float *s_g, int flags, void *stream);

/*
 * Quantize x [rows][cols] (dtype F32 or BF16, row-major) along its rows:
 * the NVFP4 form of x^T, with blocks of 16 consecutive rows of one column.
 *   codes_t  [cols][rows/2]  u8 out      scales_t [cols][rows/16] u8 out
 *   s_g      [1] fp32: out with NVFP4_SCALE_COMPUTE (the same value as for x
 *            itself: the amax does not depend on the layout), in with
 *            NVFP4_SCALE_GIVEN
 *   flags    as for nvfp4_quantize (NVFP4_FOUR_OVER_SIX allowed)
 * Bit-identical to nvfp4_quantize of a transposed copy of x, without
 * writing that copy.  These are the operands of the backward GEMMs of a
 * linear Y = X W^T in nn.Linear layout (nvfp4_gemm contracts over the
 * contiguous axis): dX = dY W takes W quantized along its rows (this call on
 * W) against dY quantized row-wise; dW = dY^T X takes dY and X quantized
 * along their rows (this call on both).  The landx.limxdynamics.com article
 * (sections on NVFP4 and on the training stage) and the d9249.github.io
 * review (section "Core idea / structure / operation") put NVFP4 on the
 * training GEMMs too; the pages do not define the recipe, so the rounding is
 * the same single RNE as everywhere else (no stochastic rounding, no
 * Hadamard transform).  cols == 0 is allowed (COMPUTE then writes s_g = 0);
 * the codes buffer serves as scratch for the amax partials.  Requires
 * rows > 0, rows % 16 == 0, rows * cols < 2^40.
 */
nvfp4_status_t nvfp4_quantize_transposed(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                         uint8_t *codes_t, uint8_t *scales_t, float *s_g, int flags,
                                         void *stream);

/*
 * adaLN fused into the quantizer: quantize y [rows][k] to NVFP4 without
 * writing y, where for row r in group g = r / rows_per_group
 *   y[r][d] = (x[r][d] - mu_r) / sqrt(var_r + eps) * (1 + scale[g][d]) + shift[g][d],
 *   mu_r, var_r the mean and biased variance of row r of x,
 * computed in fp32 (row sums in a fixed order: deterministic).
 *   x       [rows][k] dtype F32 or BF16, the pre-norm activations (tokens x
 *           hidden), shift / scale fp32 [ceil(rows / rows_per_group)][k]
 *           (one modulation per group of tokens, e.g. per frame chunk)
 *   codes   [rows][k/2] u8 out      scales [rows][k/16] u8 out
 *   s_g     [1] fp32: out with NVFP4_SCALE_COMPUTE (RN(max|y| / 2688)), in
 *           with NVFP4_SCALE_GIVEN
 * The codes equal nvfp4_quantize of y as computed here; against the exact
 * (real-number) y they can differ only where an element or a block maximum
 * lies within fp32 rounding of a decision boundary.  The yourai.pro page lists
 * a unified RoPE + adaLN kernel among the NVFP4 inference-path
 * optimizations; this is its adaLN half, fused with the activation
 * quantization that follows it (the modulated activation never goes to HBM).
 * Two passes over x (amax, then encode), the amax partials kept in the codes
 * buffer.  flags: NVFP4_SCALE_COMPUTE or NVFP4_SCALE_GIVEN only (no
 * FourOverSix here).  Requires k % 16 == 0, 16 <= k <= 4096, rows < 2^33, rows_per_group >= 1,
 * 0 <= eps finite; shift and scale 16-byte aligned.  rows == 0 is allowed
 * (COMPUTE then writes s_g = 0).
 */
nvfp4_status_t nvfp4_adaln_quantize(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t k, const float *shift,
                                    const float *scale, int64_t rows_per_group, float eps, uint8_t *codes,
                                    uint8_t *scales, float *s_g, int flags, void *stream);

/*
 * Dequantize: y[r][i] = RN_ydtype(val(code) * val(scale) * s_g), y [rows][k]
 * of dtype F32 or BF16 (one rounding of the exact product).  Same shape
 * rules as nvfp4_quantize.  Per the d9249.github.io review (dequantization
 * kernel restoring NVFP4 data) and the yourai.pro page (faster FP4
 * dequantization).
 */
nvfp4_status_t nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *s_g,
                                int64_t rows, int64_t k, void *y, nvfp4_dtype_t y_dtype, void *stream);

/*
 * W4A4 GEMM, the nn.Linear convention C = A . B^T:
 *   A [M][K] as (a_codes [M][K/2], a_scales [M][K/16], a_sg [1])
 *   B [N][K] as (b_codes [N][K/2], b_scales [N][K/16], b_sg [1])
 *   C [M][N] row-major, dtype F32 or BF16:
 *   C[m][n] = RN_cdtype(a_sg * b_sg * sum_k val(qA)val(sA) * val(qB)val(sB))
 * Each decoded element val(q)*val(s) is exact in fp16; products are summed
 * by fp16 MFMA in fp32 (order unspecified, deterministic), then scaled.
 * Per the arXiv abstract and the landx blog (section on NVFP4: GEMMs on
 * 4-bit weights and activations).  Requires M, N > 0, K > 0, K % 16 == 0,
 * M, N < 2^31.
 */
nvfp4_status_t nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_sg,
                          const uint8_t *b_codes, const uint8_t *b_scales, const float *b_sg,
                          int64_t M, int64_t N, int64_t K, void *c, nvfp4_dtype_t c_dtype, void *stream);

/*
 * Activation-quantizing linear: quantize A (a_dtype F32 or BF16, [M][K]) to
 * NVFP4, then C = A_q . B^T as in nvfp4_gemm.
 *   flags NVFP4_SCALE_COMPUTE: a_sg [1] is an output, RN_f32(max |A| / 2688);
 *   flags NVFP4_SCALE_GIVEN:   a_sg [1] is an input, e.g. written earlier on the
 *         stream by nvfp4_global_scale (the scale never leaves the device);
 *   a_codes [M][K/2], a_scales [M][K/16]: the packed activation, outputs,
 *         bit-identical to nvfp4_quantize with the same flags and a_sg;
 *   flags may add NVFP4_FOUR_OVER_SIX (the activation's block scaling).
 * The packed activation is required, not optional: the GEMM reads it back (from
 * L2 / MALL) and the library allocates nothing, so the caller owns that memory.
 * One call enqueues, on `stream`, amax and finalize kernels (COMPUTE only), the
 * encode kernel and the GEMM.  Per the arXiv abstract (W4A4 NVFP4 linears) and
 * the yourai.pro page (reduced KV-cache synchronization: scales stay on the
 * device).  Shape rules of nvfp4_gemm; unknown flags give NVFP4_ERR_FLAGS.
 */
nvfp4_status_t nvfp4_gemm_fused_act(const void *a, nvfp4_dtype_t a_dtype, int64_t M, int64_t K, float *a_sg,
                                    uint8_t *a_codes, uint8_t *a_scales, const uint8_t *b_codes,
                                    const uint8_t *b_scales, const float *b_sg, int64_t N, void *c,
                                    nvfp4_dtype_t c_dtype, int flags, void *stream);

/*
 * NVFP4 KV cache quantize: kv [heads][tokens][head_dim] bf16 ->
 *   codes [heads][tokens][head_dim/2], scales [heads][tokens][head_dim/16],
 *   head_scales [heads] fp32 (one s_g per head, from that head's amax).
 * Blocks of 16 run along head_dim.  Per the arXiv abstract (KV cache
 * quantized into NVFP4) and the d9249.github.io review (Table 3: NVFP4 KV
 * cache lowers peak memory).  Requires heads > 0, tokens >= 0,
 * head_dim % 16 == 0.
 */
nvfp4_status_t kv_quantize(const void *kv, int64_t heads, int64_t tokens, int64_t head_dim,
                           uint8_t *codes, uint8_t *scales, float *head_scales, void *stream);

/*
 * kv_quantize with FourOverSix block scaling (NVFP4_FOUR_OVER_SIX): the same
 * per-head scales, and per block the better of the two candidate scale bytes.
 * Same arguments and rules as kv_quantize.  The pages pair the FourOverSix
 * backend with the NVFP4 inference path (d9249.github.io review); its use on
 * the KV cache is this library's reading.
 */
nvfp4_status_t kv_quantize_four_over_six(const void *kv, int64_t heads, int64_t tokens, int64_t head_dim,
                                         uint8_t *codes, uint8_t *scales, float *head_scales, void *stream);

/*
 * Append to an NVFP4 KV cache in place: kv_new [heads][tokens_new][head_dim]
 * bf16 is quantized with the per-head scales already in head_scales [heads]
 * (frozen, e.g. from kv_quantize of the first chunk or from
 * nvfp4_global_scale) and written to rows token_offset .. token_offset +
 * tokens_new - 1 of each head of the cache codes [heads][cache_tokens]
 * [head_dim/2] and scales [heads][cache_tokens][head_dim/16]; every other
 * byte of the cache is left as it is.  Values beyond 2688 * head_scales[h]
 * saturate (code 6 under scale 448).  Per the yourai.pro page (in-place
 * updates of the quantized cache among the NVFP4 inference-path
 * optimizations) and the arXiv abstract (NVFP4 KV cache).  Requires
 * head_dim % 16 == 0, 0 <= token_offset, token_offset + tokens_new <=
 * cache_tokens; tokens_new == 0 is a no-op.
 */
nvfp4_status_t kv_quantize_append(const void *kv_new, int64_t heads, int64_t tokens_new, int64_t head_dim,
                                  const float *head_scales, uint8_t *codes, uint8_t *scales,
                                  int64_t cache_tokens, int64_t token_offset, void *stream);

/*
 * Rotary position embedding fused into the KV append: new keys k_new
 * [heads][tokens_new][head_dim] bf16 are rotated and quantized into rows
 * token_offset .. token_offset + tokens_new - 1 of each head of the cache
 * (codes [heads][cache_tokens][head_dim/2], scales [heads][cache_tokens]
 * [head_dim/16]) under the frozen per-head scales in head_scales [heads],
 * as kv_quantize_append does for unrotated rows.  For new token t at
 * position p = positions[t] (device int32 [tokens_new]; NULL: p =
 * token_offset + t) and each pair of adjacent dims (2i, 2i + 1):
 *   (y_2i, y_2i+1) = (x_2i cos(p th_i) - x_2i+1 sin(p th_i),
 *                     x_2i sin(p th_i) + x_2i+1 cos(p th_i)),  th_i = rope_base^(-2i / head_dim).
 * The angle p th_i is formed and reduced to [-pi, pi] in fp64; the sine,
 * cosine and rotation are fp32.  Against the exact rotation the codes can
 * differ only where an element or a block maximum lies within that fp32
 * error of a decision boundary.  The yourai.pro page lists a unified RoPE +
 * adaLN kernel and in-place updates of the quantized cache among the NVFP4
 * inference-path optimizations; this is the RoPE half, fused with the append
 * (the rotated keys never go to HBM in bf16).  Requires head_dim % 16 == 0
 * and 256 % (head_dim / 8) == 0 (head_dim 16 .. 2048, powers of two), a
 * finite rope_base > 0, 0 <= token_offset, token_offset + tokens_new <=
 * cache_tokens; tokens_new == 0 is a no-op.
 */
nvfp4_status_t kv_rope_quantize_append(const void *k_new, int64_t heads, int64_t tokens_new, int64_t head_dim,
                                       const int32_t *positions, float rope_base, const float *head_scales,
                                       uint8_t *codes, uint8_t *scales, int64_t cache_tokens,
                                       int64_t token_offset, void *stream);

/*
 * NVFP4 KV cache dequantize to bf16 [heads][tokens][head_dim]:
 *   out = RN_bf16(val(code) * val(scale) * head_scales[h]).
 * The "parallel dequantization" of the d9249.github.io review (section
 * "Core idea / structure / operation").
 */
nvfp4_status_t kv_dequantize(const uint8_t *codes, const uint8_t *scales, const float *head_scales,
                             int64_t heads, int64_t tokens, int64_t head_dim, void *kv_out,
                             void *stream);

/*
 * Softmax attention of bf16 queries over an NVFP4 KV cache, read packed:
 *   q   [heads][q_tokens][head_dim] bf16,  out [heads][q_tokens][head_dim] bf16;
 *   K, V caches as written by kv_quantize / kv_quantize_append:
 *   codes [heads][cache_tokens][head_dim/2], scales [heads][cache_tokens]
 *   [head_dim/16], per-head scales [heads]; the first kv_tokens rows of every
 *   head are attended (no mask inside them):
 *     out[h][i] = RN_bf16(sum_j w_j v_j / sum_j w_j),
 *     w_j = exp(softmax_scale * (q_i . k_j) - max_j(...)),
 *   k_j, v_j the dequantized rows val(q) val(s_b) s_g.  Computed with exact
 *   bf16 / fp16 operands on the matrix cores, fp32 accumulation and an online
 *   softmax; the probabilities are rounded to fp16 for the second product.
 *   Per the d9249.github.io review (the NVFP4 KV cache is restored by a
 *   parallel dequantization kernel for the attention) and the arXiv abstract
 *   (NVFP4 KV cache).  Requires head_dim == 128, 1 <= kv_tokens <=
 *   cache_tokens < 2^31, a finite softmax_scale; q_tokens == 0 is a no-op.
 *   workspace: optional device memory (16-byte aligned, owned by the caller,
 *   contents ignored and overwritten) of workspace_bytes bytes.  With at least
 *   kv_attention_workspace_size() bytes the cache is split across more
 *   workgroups when that balances the GPU better (fp32 partial results merged
 *   by a second kernel); with less, or NULL, the split is limited to what fits
 *   (none at 0).  Calls that share a workspace must not overlap.
 */
nvfp4_status_t kv_attention(const void *q, int64_t heads, int64_t q_tokens, int64_t head_dim,
                            const uint8_t *k_codes, const uint8_t *k_scales, const float *k_head_scales,
                            const uint8_t *v_codes, const uint8_t *v_scales, const float *v_head_scales,
                            int64_t cache_tokens, int64_t kv_tokens, float softmax_scale, void *out,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_attention for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * without the workspace, the same kernels and results as kv_attention with a
 * workspace of NVFP4_NOALLOC_SCRATCH_BYTES (32 MiB).  The split-cache partial
 * results go to a fixed device array of that size inside the library, one per
 * device, held until the process ends; the call allocates nothing (its first
 * call on a device looks up that array's address there).  A cache split whose
 * partial results would exceed the array is not chosen, down to one pass that
 * needs none, so every size kv_attention accepts runs; shapes outside those
 * limits give NVFP4_ERR_SHAPE as there.  Nothing in the array needs to start
 * at zero: every call writes all the partials it reads.  All calls on one
 * device share the array: calls that overlap in time on one device (different
 * streams, or several host threads) race and give wrong results; calls on one
 * stream are ordered and safe.  The stream must belong to a device the
 * library can run on; NVFP4_ERR_LAUNCH if the array cannot be found there.
 */
nvfp4_status_t kv_attention_noalloc(const void *q, int64_t heads, int64_t q_tokens, int64_t head_dim,
                                    const uint8_t *k_codes, const uint8_t *k_scales, const float *k_head_scales,
                                    const uint8_t *v_codes, const uint8_t *v_scales, const float *v_head_scales,
                                    int64_t cache_tokens, int64_t kv_tokens, float softmax_scale, void *out,
                                    void *stream);

/*
 * Workspace bytes at which kv_attention takes its preferred cache split for
 * these sizes on the current device (0 if it would not split), written to
 * *bytes.  Same shape rules as kv_attention (cache_tokens not needed).
 */
nvfp4_status_t kv_attention_workspace_size(int64_t heads, int64_t q_tokens, int64_t head_dim,
                                           int64_t kv_tokens, size_t *bytes);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H_ */
