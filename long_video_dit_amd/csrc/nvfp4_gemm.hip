// W4A4 NVFP4 GEMM for gfx950: C[M][N] = s_gA s_gB * sum_k a_k b_k with
// a_k = val(qA) val(sA), b_k = val(qB) val(sB), the nn.Linear convention
// (A [M][K], B [N][K], both K-contiguous).
//
// Decode path.  A decoded element val(q) * val(s) has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16; products of two are
// exact in fp32.  Packed codes and scale bytes are staged through LDS; each
// wave decodes its MFMA operands in registers (v_cvt_scalef32_pk_f16_fp4,
// then v_pk_mul_f16 by the E4M3 scale) and accumulates with
// v_mfma_f32_32x32x16_f16.  The epilogue multiplies by s_gA * s_gB and rounds
// once to the output type.  Accumulation order is fixed: deterministic.
//
// gfx950's block-scaled FP4 MFMA takes power-of-two (E8M0) scales per 32
// elements, which cannot represent E4M3 scales per 16 exactly, so it is not
// used.
//
// Tiling.  256 x 256 output tile per 256-thread workgroup (4 waves in 2 x 2,
// 128 x 128 per wave = 4 x 4 MFMA tiles of 32 x 32), K in chunks of 128,
// double-buffered LDS (72 KB).  Within a chunk the K order is permuted the
// same way for A and B: lane half h of k16-step t of sub-chunk s carries
// k = 64 s + 32 h + 8 t + (0..7), so every lane reads its 32 codes of a
// sub-chunk with one 16-byte LDS read.  Workgroup ids are remapped so that
// consecutive tiles land on the same XCD (ids are dealt round-robin over the
// 8 XCDs), then grouped 8 tile-rows high for L2 reuse.
#include <hip/hip_runtime.h>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kBM = 256, kBN = 256, kKC = 128;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

struct GemmSmem {
  uint4 a_codes[2][4 * 256];  // [stage][plane q = 2 s + h][row] 16 B
  uint4 b_codes[2][4 * 256];
  uint2 a_scales[2][256];     // [stage][row] the chunk's 8 scale bytes
  uint2 b_scales[2][256];
};

struct Staged {
  uint4 a[4], b[4];
  uint2 sa, sb;
};

// 16 bytes of codes of row `row` at byte offset `off` in the row; zero past K.
template <bool kFast>
__device__ __forceinline__ uint4 load_codes(const uint8_t* __restrict__ p, int64_t row, int64_t rows, int K,
                                            int off) {
  if (row >= rows) return make_uint4(0, 0, 0, 0);
  const uint8_t* src = p + row * (int64_t)(K / 2) + off;
  if constexpr (kFast) {
    return *reinterpret_cast<const uint4*>(src);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const int byte = off + 4 * i + b;
        if (2 * byte < K) v |= (uint32_t)src[4 * i + b] << (8 * b);
      }
      w[i] = v;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <bool kFast>
__device__ __forceinline__ uint2 load_scales(const uint8_t* __restrict__ p, int64_t row, int64_t rows, int K,
                                             int kc) {
  if (row >= rows) return make_uint2(0, 0);
  const uint8_t* src = p + row * (int64_t)(K / 16) + kc * 8;
  if constexpr (kFast) {
    return *reinterpret_cast<const uint2*>(src);
  } else {
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int b = 0; b < 8; b++)
      if (kc * kKC + 16 * b < K) w[b / 4] |= (uint32_t)src[b] << (8 * (b % 4));
    return make_uint2(w[0], w[1]);
  }
}

template <bool kFast>
__device__ __forceinline__ void load_chunk(Staged& st, const uint8_t* __restrict__ a_codes,
                                           const uint8_t* __restrict__ a_scales, const uint8_t* __restrict__ b_codes,
                                           const uint8_t* __restrict__ b_scales, int64_t m0, int64_t n0, int M, int N,
                                           int K, int kc) {
  const int t = threadIdx.x;
  const int q = t & 3;
  const int off = kc * (kKC / 2) + 16 * q;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int row = (t >> 2) + 64 * i;
    st.a[i] = load_codes<kFast>(a_codes, m0 + row, M, K, off);
    st.b[i] = load_codes<kFast>(b_codes, n0 + row, N, K, off);
  }
  st.sa = load_scales<kFast>(a_scales, m0 + t, M, K, kc);
  st.sb = load_scales<kFast>(b_scales, n0 + t, N, K, kc);
}

__device__ __forceinline__ void store_chunk(const Staged& st, GemmSmem& sm, int stage) {
  const int t = threadIdx.x;
  const int q = t & 3;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int row = (t >> 2) + 64 * i;
    sm.a_codes[stage][q * 256 + row] = st.a[i];
    sm.b_codes[stage][q * 256 + row] = st.b[i];
  }
  sm.a_scales[stage][t] = st.sa;
  sm.b_scales[stage][t] = st.sb;
}

// 8 E2M1 codes (one 32-bit word, element e in bits 4e+3..4e) times an fp16
// scale -> 8 exact fp16 values.
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16x2 sc) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ f16x2 scale_f16x2(uint32_t byte) {
  const _Float16 v = (_Float16)e4m3_value(byte);  // exact: E4M3 values fit fp16
  return f16x2{v, v};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int t) {
  return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}

// Workgroup id -> (tile_m, tile_n): XCD-contiguous, then grouped by 8 tile rows.
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b % kXcds, idx = b / kXcds;
  const int q = T / kXcds, r = T % kXcds;
  const int lin = xcd * q + (xcd < r ? xcd : r) + idx;
  const int per_group = kGroupM * tiles_n;
  const int group = lin / per_group;
  const int first_m = group * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in_group = lin % per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

template <bool kFast, bool kBf16Out>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_sg,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, const float* __restrict__ b_sg, int M,
    int N, int K, void* __restrict__ c, int tiles_m, int tiles_n) {
  __shared__ GemmSmem sm;
  int tm, tn;
  tile_of(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int nk = (K + kKC - 1) / kKC;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x16{};

  Staged st;
  load_chunk<kFast>(st, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, 0);
  store_chunk(st, sm, 0);
  if (nk > 1) load_chunk<kFast>(st, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, 1);
  __syncthreads();

  for (int kc = 0; kc < nk; kc++) {
    const int cur = kc & 1;
    if (kc + 1 < nk) store_chunk(st, sm, cur ^ 1);
    if (kc + 2 < nk) load_chunk<kFast>(st, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, kc + 2);
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int q = 2 * s + h;
      uint4 ca[4], cb[4];
      f16x2 sa_lo[4], sa_hi[4], sb_lo[4], sb_hi[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = wm * 128 + 32 * i + r;
        ca[i] = sm.a_codes[cur][q * 256 + row];
        const uint2 s8 = sm.a_scales[cur][row];
        const uint32_t pair = ((q < 2 ? s8.x : s8.y) >> (16 * (q & 1))) & 0xffffu;
        sa_lo[i] = scale_f16x2(pair & 0xffu);
        sa_hi[i] = scale_f16x2(pair >> 8);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = wn * 128 + 32 * j + r;
        cb[j] = sm.b_codes[cur][q * 256 + row];
        const uint2 s8 = sm.b_scales[cur][row];
        const uint32_t pair = ((q < 2 ? s8.x : s8.y) >> (16 * (q & 1))) & 0xffffu;
        sb_lo[j] = scale_f16x2(pair & 0xffu);
        sb_hi[j] = scale_f16x2(pair >> 8);
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        f16x8 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) av[i] = decode8(word_of(ca[i], t), t < 2 ? sa_lo[i] : sa_hi[i]);
#pragma unroll
        for (int j = 0; j < 4; j++) bv[j] = decode8(word_of(cb[j], t), t < 2 ? sb_lo[j] : sb_hi[j]);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Epilogue: lane (r, h), accumulator element e is row 8 (e / 4) + 4 h + e % 4,
  // column r of the 32 x 32 tile.
  const float g = a_sg[0] * b_sg[0];
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t col = n0 + wn * 128 + 32 * j + r;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
        if (row < M && col < N) {
          const float v = acc[i][j][e] * g;
          if constexpr (kBf16Out)
            reinterpret_cast<__bf16*>(c)[row * N + col] = (__bf16)v;
          else
            reinterpret_cast<float*>(c)[row * N + col] = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_sg, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_sg, int64_t M, int64_t N, int64_t K, void* c,
                       int c_dtype, hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kGemmThreads);
  const bool fast = (K % kKC == 0) && ((uintptr_t)a_codes % 16 == 0) && ((uintptr_t)b_codes % 16 == 0) &&
                    ((uintptr_t)a_scales % 8 == 0) && ((uintptr_t)b_scales % 8 == 0);
  const bool bf = c_dtype == kDtypeBf16;
#define NVFP4_GEMM_LAUNCH(F, B)                                                                                    \
  launch_kernel(gemm_w4a4_kernel<F, B>, grid, block, 0, stream, a_codes, a_scales, a_sg, b_codes, b_scales, b_sg, \
                (int)M, (int)N, (int)K, c, tiles_m, tiles_n)
  if (fast) return bf ? NVFP4_GEMM_LAUNCH(true, true) : NVFP4_GEMM_LAUNCH(true, false);
  return bf ? NVFP4_GEMM_LAUNCH(false, true) : NVFP4_GEMM_LAUNCH(false, false);
#undef NVFP4_GEMM_LAUNCH
}

}  // namespace nvfp4
