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
// Two kernels share that decode and MFMA code.  Both take a 256 x 256 output
// tile per 256-thread workgroup (4 waves in 2 x 2, 128 x 128 per wave = 4 x 4
// MFMA tiles of 32 x 32; the fast kernel also 256 x 192, 4 x 3 per wave);
// within a stage the K order is permuted the same way
// for A and B: lane half h of k16-step t of sub-chunk s carries
// k = 64 s + 32 h + 8 t + (0..7), so every lane reads its 32 codes of a
// sub-chunk with one 16-byte LDS read.
//   gemm_w4a4_fast_kernel (K % 512 == 0, aligned operands): persistent, one
//     workgroup per CU walking its tiles; stages of K = 256 copied global ->
//     LDS by the DMA path (global_load_lds_dwordx4), two stages plus a 16 KB
//     epilogue buffer in the 160 KB of LDS; hand-interleaved MFMA / decode
//     steps; each tile starts with zero-accumulator MFMAs instead of zeroing
//     its accumulators.
//   gemm_w4a4_kernel (any K % 16 == 0, any alignment): one tile per
//     workgroup, register-staged stages of K = 128, double-buffered LDS
//     (72 KB), zero-filled K tails.
// Workgroup ids (fast kernel: tile indices) are remapped so that consecutive
// tiles land on the same XCD (ids are dealt round-robin over the 8 XCDs),
// then grouped 8 tile-rows high for L2 reuse.
#include <hip/hip_runtime.h>
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

#ifndef NVFP4_GEMM_WM
#define NVFP4_GEMM_WM 2
#define NVFP4_GEMM_WN 2
#endif

namespace nvfp4 {

namespace {

constexpr int kTile = 256;  // rows of A and of B per workgroup tile
constexpr int kKC = 128;    // K per LDS stage
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

// LDS planes are padded by 64 B so that the 16-byte stores of 4 threads
// sharing a row (one per plane) and the 16-byte operand reads of 16
// consecutive rows both spread over all 64 banks.
constexpr int kPlaneStride = kTile + 4;  // uint4 units

struct GemmSmem {
  uint4 a_codes[2][4 * kPlaneStride];  // [stage][plane q = 2 s + h][row] 16 B
  uint4 b_codes[2][4 * kPlaneStride];
  uint32_t a_scales[2][4][kTile];      // [stage][q][row] fp16 scales of blocks 2q, 2q+1
  uint32_t b_scales[2][4][kTile];
};

// Wave layout: WM x WN waves, each FM x FN MFMA tiles of 32 x 32, covering
// the 256 x 256 workgroup tile.
template <int WM, int WN>
struct GemmCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int FM = kTile / (32 * WM);
  static constexpr int FN = kTile / (32 * WN);
  static constexpr int kPieces = 4 * kTile / kThreads;  // 16-byte code pieces per thread per operand
  static constexpr int kScaleRows = 2 * kTile / kThreads;  // scale rows (A then B) per thread
};

template <typename C>
struct Staged {
  uint4 a[C::kPieces], b[C::kPieces];
  uint2 s[C::kScaleRows];
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

// The 8 scale bytes of chunk kc of row `row`; zero past K.
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

// Global -> registers for chunk kc: thread t loads 16-byte pieces
// (row = p / 4, plane q = p % 4) for p = t + kThreads * i, which gives four
// consecutive threads 64 contiguous bytes of a row.
template <typename C, bool kFast>
__device__ __forceinline__ void load_chunk(Staged<C>& st, const uint8_t* __restrict__ a_codes,
                                           const uint8_t* __restrict__ a_scales, const uint8_t* __restrict__ b_codes,
                                           const uint8_t* __restrict__ b_scales, int64_t m0, int64_t n0, int M, int N,
                                           int K, int kc) {
  const int t = threadIdx.x;
  const int q = t & 3;
  const int off = kc * (kKC / 2) + 16 * q;
#pragma unroll
  for (int i = 0; i < C::kPieces; i++) {
    const int row = (t >> 2) + (C::kThreads / 4) * i;
    st.a[i] = load_codes<kFast>(a_codes, m0 + row, M, K, off);
    st.b[i] = load_codes<kFast>(b_codes, n0 + row, N, K, off);
  }
#pragma unroll
  for (int i = 0; i < C::kScaleRows; i++) {
    const int row = t + C::kThreads * i;  // 0..255: A rows, 256..511: B rows
    st.s[i] = row < kTile ? load_scales<kFast>(a_scales, m0 + row, M, K, kc)
                          : load_scales<kFast>(b_scales, n0 + row - kTile, N, K, kc);
  }
}

// Two E4M3 scale bytes -> two exact fp16 values: the byte shifted into an
// fp16 bit pattern (exponent bits 6:3 -> 14:10, mantissa -> 9:7) reads as
// 2^-8 times the E4M3 value, subnormals included; one packed multiply by 256
// restores it.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t b0, uint32_t b1) {
  const f16x2 v = __builtin_bit_cast(f16x2, (b0 << 7) | (b1 << 23)) * f16x2{(_Float16)256.0f, (_Float16)256.0f};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename C>
__device__ __forceinline__ void store_chunk(const Staged<C>& st, GemmSmem& sm, int stage) {
  const int t = threadIdx.x;
  const int q = t & 3;
#pragma unroll
  for (int i = 0; i < C::kPieces; i++) {
    const int row = (t >> 2) + (C::kThreads / 4) * i;
    sm.a_codes[stage][q * kPlaneStride + row] = st.a[i];
    sm.b_codes[stage][q * kPlaneStride + row] = st.b[i];
  }
#pragma unroll
  for (int i = 0; i < C::kScaleRows; i++) {
    const int row = t + C::kThreads * i;
    uint32_t(*dst)[kTile] = row < kTile ? sm.a_scales[stage] : sm.b_scales[stage];
    const int rr = row & (kTile - 1);
    const uint32_t w[2] = {st.s[i].x, st.s[i].y};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t b = w[j / 2] >> (16 * (j & 1));
      dst[j][rr] = e4m3x2_to_f16x2(b & 0xffu, (b >> 8) & 0xffu);
    }
  }
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

__device__ __forceinline__ uint32_t word_of(const uint4& v, int t) {
  return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}

// Linear tile index -> (tile_m, tile_n), grouped by kGroupM tile rows so
// that consecutive indices share A rows and B rows.
__device__ __forceinline__ void tile_of_lin(int lin, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int group = lin / per_group;
  const int first_m = group * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in_group = lin % per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
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

template <int WM, int WN, bool kFast, bool kBf16Out>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_sg,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, const float* __restrict__ b_sg, int M,
    int N, int K, void* __restrict__ c, int tiles_m, int tiles_n) {
  using C = GemmCfg<WM, WN>;
  constexpr int FM = C::FM, FN = C::FN;
  __shared__ GemmSmem sm;
  int tm, tn;
  tile_of(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
  const int nk = (K + kKC - 1) / kKC;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, h = lane >> 5;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = f32x16{};

  Staged<C> st;
  load_chunk<C, kFast>(st, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, 0);
  store_chunk<C>(st, sm, 0);
  if (nk > 1) load_chunk<C, kFast>(st, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, 1);
  __syncthreads();

  for (int kc = 0; kc < nk; kc++) {
    const int cur = kc & 1;
    if (kc + 1 < nk) store_chunk<C>(st, sm, cur ^ 1);
    if (kc + 2 < nk) load_chunk<C, kFast>(st, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, kc + 2);
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int q = 2 * s + h;
      uint4 ca[FM], cb[FN];
      f16x2 sa[FM], sb[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) {
        const int row = wm * (32 * FM) + 32 * i + r;
        ca[i] = sm.a_codes[cur][q * kPlaneStride + row];
        sa[i] = __builtin_bit_cast(f16x2, sm.a_scales[cur][q][row]);
      }
#pragma unroll
      for (int j = 0; j < FN; j++) {
        const int row = wn * (32 * FN) + 32 * j + r;
        cb[j] = sm.b_codes[cur][q * kPlaneStride + row];
        sb[j] = __builtin_bit_cast(f16x2, sm.b_scales[cur][q][row]);
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        f16x8 av[FM], bv[FN];
#pragma unroll
        for (int i = 0; i < FM; i++) {
          const _Float16 sc = t < 2 ? sa[i].x : sa[i].y;
          av[i] = decode8(word_of(ca[i], t), f16x2{sc, sc});
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
          const _Float16 sc = t < 2 ? sb[j].x : sb[j].y;
          bv[j] = decode8(word_of(cb[j], t), f16x2{sc, sc});
        }
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
          for (int j = 0; j < FN; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Epilogue: lane (r, h), accumulator element e is row 8 (e / 4) + 4 h + e % 4,
  // column r of the 32 x 32 tile.
  const float g = a_sg[0] * b_sg[0];
#pragma unroll
  for (int i = 0; i < FM; i++) {
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int64_t col = n0 + wn * (32 * FN) + 32 * j + r;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int64_t row = m0 + wm * (32 * FM) + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
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

// ---------------------------------------------------------------------------
// Fast path (K % 512 == 0, N % 4 == 0, aligned operands): the packed operands
// go global -> LDS with global_load_lds_dwordx4 (no register staging, no LDS
// stores), two LDS stages of K = 256 held in two distinct LDS objects so the
// compiler can tell the prefetch of one stage from the reads of the other.
// Per stage and operand: codes [256 rows][8 slots of 16 B] (256 codes per
// row) with slot = plane q ^ ((row / 2) % 8), which makes both the 128 B
// per-row coalesced fills and the 16-row operand reads bank-conflict free;
// raw scale bytes [256 rows][16 B].  The MFMA takes B as its first operand,
// so every lane ends with 4 consecutive output columns of one row and the
// epilogue stores 8 (bf16) or 16 (fp32) bytes per instruction.  Rows past M
// or N are clamped to the last row: they only feed outputs that are never
// stored.
//
// The k16-steps of all stages and tiles of a workgroup form one software
// pipeline: each step's MFMAs run interleaved with the decode of the next
// step, also across stage and tile boundaries, so no stage starts with a
// decode or a scale conversion that the matrix cores would wait for.
typedef __attribute__((address_space(3))) void lds_void_t;

// global -> LDS copy of 16 bytes per lane: lane i reads base + voff[i] and
// writes LDS address lds + 16 i; lds and base are
// wave-uniform (M0 and an SGPR pair).  Issued as asm statements without
// outputs so that the compiler does not track these LDS writes (its tracking
// falls back to waiting for every outstanding copy before any LDS read, which
// would serialize the prefetch); completion is enforced explicitly with
// s_waitcnt vmcnt(0) + s_barrier before a stage is read.  M0 is reserved by
// the compiler, hence the warning pragma: the fast kernel contains no
// compiler-generated use of M0 (tests/test_build_checks.py verifies this on
// the generated assembly), so setting it here disturbs nothing.  The s_nop
// is the one wait state an LDS DMA needs after an SALU write of M0 (the
// compiler's hazard recognizer does not look inside asm statements).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "m0");
}
#pragma clang diagnostic pop

constexpr int kFastKC = 256;  // K per LDS stage of the fast path: 128 code bytes per row
// Where a stage's refill goes (see fast_stage): the waves synchronize after
// k16-step kBarrierStep, kRefillBurst copies follow at once, and the rest come
// one after every kRefillEvery-th MFMA block from step kRefillStep on.  On the
// FFN shapes this is ~2.5% faster than issuing all copies at the barrier; the
// matrix cores lose less time to the CU's address unit.  (6 at once and one
// after every block measured 0.5-0.7% faster than 10 at once and one after
// every other block, with the zero-accumulator tile start.)
constexpr int kBarrierStep = 11;
constexpr int kRefillStep = 12;
constexpr int kRefillBurst = 6;
constexpr int kRefillEvery = 1;

// The fast path's output tile is 256 rows of A by 64 FN rows of B: each of
// the 4 waves (2 x 2) holds 128 rows x 32 FN columns, FN = 4 (256 x 256) or
// FN = 3 (256 x 192, which tiles a 3072-column output into 16 instead of 12
// columns of tiles).  FN is the number of 32-column B fragments per wave.
template <int FN>
struct __attribute__((aligned(16))) FastStage {
  uint8_t a_codes[kTile * 128];    // [row][8 slots of 16 B], slot = plane q ^ ((row / 2) % 8)
  uint8_t b_codes[64 * FN * 128];  // the same for the 64 FN rows of B
  uint8_t a_scales[kTile * 16];    // [row][16 scale bytes]
  uint8_t b_scales[64 * FN * 16];
  // LDS byte offsets of the parts of a stage.
  static constexpr uint32_t kA = 0, kB = kTile * 128, kSA = kB + 64 * FN * 128, kSB = kSA + kTile * 16;
};

// Copies of one stage (K = 256 of the tile's A and B rows) issued by one
// thread: wave w fills A rows 64 w .. 64 w + 63 and B rows 16 FN w ..
// 16 FN w + 16 FN - 1, 8 rows (1 KiB of codes) per 16-byte copy instruction,
// and 64 rows of scale bytes (16 per row and stage, 16-byte aligned since
// K % 512 == 0) per copy: A's rows 64 w .., B's for the first FN waves.  For
// a full tile the per-lane part of each source offset only depends on the
// lane and on the instruction's parity (the plane swizzle q ^ ((row / 2) % 8)
// repeats every 16 rows), so it is kept in 3 VGPRs and the row advance goes
// into the uniform SGPR base.  Tiles that cross the last row of A or B clamp
// every lane's row and take the per-lane path.
struct FastLoad {
  uint32_t vo[2];  // code offsets of even / odd instructions (full tiles)
  uint32_t vs;     // scale row offset (full tiles)
};

__device__ __forceinline__ FastLoad fast_load_offsets(int K) {
  const int lane = threadIdx.x & 63;
  const uint32_t row_bytes = (uint32_t)(K / 2), srow_bytes = (uint32_t)(K / 16);
  FastLoad o;
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int row = 8 * p + (lane >> 3);  // row within a 16-row period
    const uint32_t q = (lane & 7) ^ ((row >> 1) & 7);
    o.vo[p] = (uint32_t)(lane >> 3) * row_bytes + 16 * q;
  }
  o.vs = (uint32_t)lane * srow_bytes;
  return o;
}

// Stage kc of the tile at rows (m0, n0) -> the LDS stage at address `lds`.
template <int FN>
__device__ __forceinline__ void fast_load_stage(uint32_t lds, const FastLoad& o, bool edge,
                                                const uint8_t* __restrict__ a_codes,
                                                const uint8_t* __restrict__ a_scales,
                                                const uint8_t* __restrict__ b_codes,
                                                const uint8_t* __restrict__ b_scales, int64_t m0, int64_t n0, int M,
                                                int N, int K, int kc) {
  using S = FastStage<FN>;
  constexpr int kCopiesB = 2 * FN;  // 8-row copies of B per wave (even: the parity rule above holds)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t row_bytes = K / 2, srow_bytes = K / 16;
  if (!edge) {
    const uint8_t* ac = a_codes + (m0 + 64 * w) * row_bytes + kc * 128;
    const uint8_t* bc = b_codes + (n0 + 16 * FN * w) * row_bytes + kc * 128;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      lds_dma16(ac + 8 * i * row_bytes, o.vo[i & 1], lds + S::kA + (uint32_t)(w * 8 + i) * 64 * 16);
      if (i < kCopiesB)
        lds_dma16(bc + 8 * i * row_bytes, o.vo[i & 1], lds + S::kB + (uint32_t)(w * kCopiesB + i) * 64 * 16);
    }
    const uint32_t d0 = (uint32_t)w * 64 * 16;
    lds_dma16(a_scales + (m0 + 64 * w) * srow_bytes + kc * 16, o.vs, lds + S::kSA + d0);
    if (FN == 4 || w < FN) lds_dma16(b_scales + (n0 + 64 * w) * srow_bytes + kc * 16, o.vs, lds + S::kSB + d0);
    return;
  }
  const uint8_t* ac = a_codes + kc * 128;
  const uint8_t* bc = b_codes + kc * 128;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    {
      const int slot0 = (w * 8 + i) * 64;
      const int row = (slot0 + lane) >> 3;
      const uint32_t q = ((slot0 + lane) & 7) ^ ((row >> 1) & 7);
      const int64_t ra = m0 + row < M ? m0 + row : M - 1;
      lds_dma16(ac, (uint32_t)(ra * row_bytes) + 16 * q, lds + S::kA + (uint32_t)slot0 * 16);
    }
    if (i < kCopiesB) {
      const int slot0 = (w * kCopiesB + i) * 64;
      const int row = (slot0 + lane) >> 3;
      const uint32_t q = ((slot0 + lane) & 7) ^ ((row >> 1) & 7);
      const int64_t rb = n0 + row < N ? n0 + row : N - 1;
      lds_dma16(bc, (uint32_t)(rb * row_bytes) + 16 * q, lds + S::kB + (uint32_t)slot0 * 16);
    }
  }
  const int row = 64 * w + lane;
  const int64_t ra = m0 + row < M ? m0 + row : M - 1;
  const uint32_t d0 = (uint32_t)w * 64 * 16;
  lds_dma16(a_scales + kc * 16, (uint32_t)(ra * srow_bytes), lds + S::kSA + d0);
  if (FN == 4 || w < FN) {
    const int64_t rb = n0 + row < N ? n0 + row : N - 1;
    lds_dma16(b_scales + kc * 16, (uint32_t)(rb * srow_bytes), lds + S::kSB + d0);
  }
}

// The copies of one stage issued one at a time, so that part of a refill can
// be spread between MFMA blocks: issued in one burst, the 4 waves' 18 copies
// keep the CU's address unit busy ~1300 cycles, during which the matrix cores
// wait.  copy<k>() issues this wave's copy k of fast_load_stage's full-tile
// path (k < 8: A codes, then 2 FN B codes, then A's and B's scale rows) from
// sources and LDS destinations set up once per stage; burst<n>() copies
// 0 .. n - 1.  A tile that crosses row M or column N has its stage issued
// whole (whole_stage()) instead.
template <int FN>
struct FastRefill {
  static constexpr int kCopies = 8 + 2 * FN + 2;
  const uint8_t *ac, *bc, *as, *bs;  // this wave's sources of copy 0 of each kind
  int64_t row8;                      // 8 rows of codes in bytes
  uint32_t la, lb, lsa, lsb;         // this wave's LDS destinations of copy 0 of each kind
  FastLoad o;
  bool split, split_sb;              // full tile: copies one at a time (B scales: only the first FN waves)
  bool whole;                        // edge tile: the stage in one go, with the arguments below
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  int64_t m0, n0;
  int M, N, K, kc;
  uint32_t lds;

  __device__ __forceinline__ FastRefill(uint32_t lds_, const FastLoad& o_, bool on, bool edge,
                                        const uint8_t* __restrict__ a_codes_, const uint8_t* __restrict__ a_scales_,
                                        const uint8_t* __restrict__ b_codes_, const uint8_t* __restrict__ b_scales_,
                                        int64_t m0_, int64_t n0_, int M_, int N_, int K_, int kc_)
      : o(o_), a_codes(a_codes_), a_scales(a_scales_), b_codes(b_codes_), b_scales(b_scales_), m0(m0_), n0(n0_),
        M(M_), N(N_), K(K_), kc(kc_), lds(lds_) {
    using S = FastStage<FN>;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row_bytes = K / 2, srow_bytes = K / 16;
    split = on && !edge;
    split_sb = split && (FN == 4 || w < FN);
    whole = on && edge;
    row8 = 8 * row_bytes;
    ac = a_codes + (m0 + 64 * w) * row_bytes + kc * 128;
    bc = b_codes + (n0 + 16 * FN * w) * row_bytes + kc * 128;
    as = a_scales + (m0 + 64 * w) * srow_bytes + kc * 16;
    bs = b_scales + (n0 + 64 * w) * srow_bytes + kc * 16;
    la = lds + S::kA + (uint32_t)(w * 8) * 64 * 16;
    lb = lds + S::kB + (uint32_t)(w * 2 * FN) * 64 * 16;
    lsa = lds + S::kSA + (uint32_t)w * 64 * 16;
    lsb = lds + S::kSB + (uint32_t)w * 64 * 16;
  }

  __device__ __forceinline__ void whole_stage() const {
    if (whole) fast_load_stage<FN>(lds, o, true, a_codes, a_scales, b_codes, b_scales, m0, n0, M, N, K, kc);
  }

  template <int n, int k = 0>
  __device__ __forceinline__ void burst() const {
    if constexpr (k < n) {
      copy<k>();
      burst<n, k + 1>();
    }
  }

  template <int k>
  __device__ __forceinline__ void copy() const {
    if constexpr (k < 8) {
      if (split) lds_dma16(ac + k * row8, o.vo[k & 1], la + (uint32_t)k * 64 * 16);
    } else if constexpr (k < 8 + 2 * FN) {
      constexpr int i = k - 8;
      if (split) lds_dma16(bc + i * row8, o.vo[i & 1], lb + (uint32_t)i * 64 * 16);
    } else if constexpr (k == 8 + 2 * FN) {
      if (split) lds_dma16(as, o.vs, lsa);
    } else if constexpr (k == 9 + 2 * FN) {
      if (split_sb) lds_dma16(bs, o.vs, lsb);
    }
  }
};

// Registers that carry the pipeline from step to step: the packed codes and
// fp16 scale pairs of two sub-chunks (sub-chunk s of a stage uses buffer
// s % 2) and the decoded MFMA operands of two k16-steps (step parity).
template <int FN>
struct FastPipe {
  uint4 ca[2][4], cb[2][FN];
  uint32_t sa[2][4], sb[2][FN];
  f16x8 av[2][4], bv[2][FN];
};

// Per-lane LDS offsets of the operand reads: lane (r, h) of wave (wm, wn)
// reads rows wm * 128 + 32 i + r of A and wn * 32 FN + 32 j + r of B; within
// a row, code plane q sits in slot q ^ sw with sw = (r / 2) % 8 (the same
// for all rows of the lane, which are 4 KiB apart), and the scale bytes of
// blocks 2q, 2q + 1 at byte 2q.
struct FastLane {
  uint32_t a, b;    // code row offsets (row * 128) of row i = 0
  uint32_t sa, sb;  // scale byte offsets (row * 16 + 2 h) of row i = 0
  uint32_t hsw;     // 16 * (h ^ sw): slot offset of plane q = 2 s + h is hsw ^ (32 s)
};

// Sub-chunk s (K = 64 s .. 64 s + 63 of a stage) of LDS stage S -> buffer u:
// this lane's 16 code bytes of plane q = 2 s + h of its 4 A rows and FN B
// rows (one 16-byte read each) and the 2 scale bytes of blocks 2q, 2q + 1 of
// each row, left raw: fast_convert_scales turns them into fp16 once the reads
// have landed.  The row offsets pass through an empty asm statement so that
// the compiler derives each address here instead of keeping all of them
// (2 stages x 4 sub-chunks x 8 rows) live in registers.
template <int FN>
__device__ __forceinline__ void fast_read_sub(const FastStage<FN>& S, FastPipe<FN>& P, int u, const FastLane& L,
                                              int s) {
  uint32_t la = L.a, lb = L.b, lsa = L.sa, lsb = L.sb;
  asm volatile("" : "+v"(la), "+v"(lb), "+v"(lsa), "+v"(lsb));
  const uint32_t slot = L.hsw ^ (32u * s);
  const uint8_t* ac = S.a_codes + (la + slot);
  const uint8_t* bc = S.b_codes + (lb + slot);
  const uint8_t* as = S.a_scales + (lsa + 4 * s);
  const uint8_t* bs = S.b_scales + (lsb + 4 * s);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    P.ca[u][i] = *reinterpret_cast<const uint4*>(ac + 4096 * i);
    P.sa[u][i] = *reinterpret_cast<const uint16_t*>(as + 512 * i);
    if (i < FN) {
      P.cb[u][i] = *reinterpret_cast<const uint4*>(bc + 4096 * i);
      P.sb[u][i] = *reinterpret_cast<const uint16_t*>(bs + 512 * i);
    }
  }
}

// Two E4M3 scale bytes -> two fp16 with the hardware converter (scale 1.0).
// Exact: every finite E4M3 value, subnormals and signed zero included, is an
// fp16 value.
template <int FN>
__device__ __forceinline__ void fast_convert_scales(FastPipe<FN>& P, int u) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    P.sa[u][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(P.sa[u][i], 1.0f, false));
    if (i < FN)
      P.sb[u][i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(P.sb[u][i], 1.0f, false));
  }
}

// The first k16-step of a workgroup's pipeline (sub-chunk 0, word 0, blocks 2h).
template <int FN>
__device__ __forceinline__ void fast_decode_first(FastPipe<FN>& P) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const _Float16 sa = __builtin_bit_cast(f16x2, P.sa[0][i]).x;
    P.av[0][i] = decode8(P.ca[0][i].x, f16x2{sa, sa});
    if (i < FN) {
      const _Float16 sb = __builtin_bit_cast(f16x2, P.sb[0][i]).x;
      P.bv[0][i] = decode8(P.cb[0][i].x, f16x2{sb, sb});
    }
  }
}

// One quarter of a k16-step, hand-interleaved: 4 MFMAs (output tiles (j, 0..3)
// of B frag j against the 4 A frags) with 4 decode VALU instructions after
// each, which decode two frags (x, y) of the NEXT k16-step (4 conversions +
// 4 fp16 scale multiplies each).  The compiler schedules MFMAs back to back
// and the decode work in long runs, so a wave (one per SIMD) alternates
// between an idle matrix core and an idle VALU; this keeps both busy.  `hi`
// selects which fp16 of the scale pair applies (blocks 2q / 2q + 1).
// Register hazards: the decoded outputs are next-step buffers whose last MFMA
// readers were issued at least one MFMA (32 cycles) earlier, and every output
// is first read by an MFMA at least one block later; each block starts with
// s_nop for the VALU-write -> MFMA-read distance across blocks.
#define NVFP4_DEC_PAIR(O, W, S, SEL, OPS)                                          \
  "v_cvt_scalef32_pk_f16_fp4 %[" O "], %[" W "], 1.0" SEL "\n\t"                  \
  "v_pk_mul_f16 %[" O "], %[" S "], %[" O "]" OPS "\n\t"
// op_sel of the scale multiply: the fp16 scale of block 2q (LO) or 2q + 1 (HI)
// of the scale pair, broadcast to both halves.
#define NVFP4_OPS_LO " op_sel:[0,0] op_sel_hi:[0,1]"
#define NVFP4_OPS_HI " op_sel:[1,0] op_sel_hi:[1,1]"
#define NVFP4_MFMA_ACC(C) "v_mfma_f32_32x32x16_f16 %[" C "], %[b], %[a" C "], %[" C "]\n\t"
#define NVFP4_MFMA_ZERO(C) "v_mfma_f32_32x32x16_f16 %[" C "], %[b], %[a" C "], 0\n\t"
// Both forms of a block in one asm statement, chosen by the wave-uniform
// operand z (nonzero: zero accumulator), so that the accumulators stay tied
// to the same registers on both paths.
#define NVFP4_EITHER(BODY_ZERO, BODY_ACC)                                         \
  "s_cmp_lg_u32 %[z], 0\n\ts_cbranch_scc0 .Lacc%=\n\t" BODY_ZERO "s_branch .Lend%=\n" \
  ".Lacc%=:\n\t" BODY_ACC ".Lend%=:\n\t"

template <bool kHi, bool kMaybeZero>
__device__ __forceinline__ void mfma4_decode2(f32x16& c0, f32x16& c1, f32x16& c2, f32x16& c3, const f16x8& b,
                                              const f16x8 (&a)[4], uint32_t wx, uint32_t sx, uint32_t wy,
                                              uint32_t sy, f16x8& ox, f16x8& oy, uint32_t zero) {
  uint32_t x0, x1, x2, x3, y0, y1, y2, y3;
#define NVFP4_BODY(OPS, MF)                                                                          \
  "s_nop 1\n\t" MF("c0") NVFP4_DEC_PAIR("x0", "wx", "sx", "", OPS)                                   \
      NVFP4_DEC_PAIR("x1", "wx", "sx", " op_sel:[1,0,0]", OPS) MF("c1")                              \
      NVFP4_DEC_PAIR("x2", "wx", "sx", " op_sel:[0,1,0]", OPS)                                       \
      NVFP4_DEC_PAIR("x3", "wx", "sx", " op_sel:[1,1,0]", OPS) MF("c2")                              \
      NVFP4_DEC_PAIR("y0", "wy", "sy", "", OPS) NVFP4_DEC_PAIR("y1", "wy", "sy", " op_sel:[1,0,0]", OPS) \
      MF("c3") NVFP4_DEC_PAIR("y2", "wy", "sy", " op_sel:[0,1,0]", OPS)                              \
      NVFP4_DEC_PAIR("y3", "wy", "sy", " op_sel:[1,1,0]", OPS)
#define NVFP4_OUT2                                                                                         \
  [c0] "+a"(c0), [c1] "+a"(c1), [c2] "+a"(c2), [c3] "+a"(c3), [x0] "=&v"(x0), [x1] "=&v"(x1), [x2] "=&v"(x2), \
      [x3] "=&v"(x3), [y0] "=&v"(y0), [y1] "=&v"(y1), [y2] "=&v"(y2), [y3] "=&v"(y3)
#define NVFP4_IN2                                                                                          \
  [b] "v"(b), [ac0] "v"(a[0]), [ac1] "v"(a[1]), [ac2] "v"(a[2]), [ac3] "v"(a[3]), [wx] "v"(wx), [sx] "v"(sx), \
      [wy] "v"(wy), [sy] "v"(sy)
  if constexpr (kHi && kMaybeZero)
    asm volatile(NVFP4_EITHER(NVFP4_BODY(NVFP4_OPS_HI, NVFP4_MFMA_ZERO), NVFP4_BODY(NVFP4_OPS_HI, NVFP4_MFMA_ACC))
                 : NVFP4_OUT2 : NVFP4_IN2, [z] "s"(zero) : "scc");
  else if constexpr (kHi)
    asm volatile(NVFP4_BODY(NVFP4_OPS_HI, NVFP4_MFMA_ACC) : NVFP4_OUT2 : NVFP4_IN2);
  else if constexpr (kMaybeZero)
    asm volatile(NVFP4_EITHER(NVFP4_BODY(NVFP4_OPS_LO, NVFP4_MFMA_ZERO), NVFP4_BODY(NVFP4_OPS_LO, NVFP4_MFMA_ACC))
                 : NVFP4_OUT2 : NVFP4_IN2, [z] "s"(zero) : "scc");
  else
    asm volatile(NVFP4_BODY(NVFP4_OPS_LO, NVFP4_MFMA_ACC) : NVFP4_OUT2 : NVFP4_IN2);
#undef NVFP4_BODY
#undef NVFP4_OUT2
#undef NVFP4_IN2
  ox = __builtin_bit_cast(f16x8, u32x4{x0, x1, x2, x3});
  oy = __builtin_bit_cast(f16x8, u32x4{y0, y1, y2, y3});
}

// The same with three frags (x, y, z) decoded around the 4 MFMAs, 6 decode
// VALU instructions after each: the last block of a k16-step of a 256 x 192
// tile, which decodes the next step's 3 B frags.  The hazard rules above
// hold: the outputs' last MFMA readers are the previous step's blocks, and
// their first readers come in the next step's blocks, after its s_nop.
template <bool kHi, bool kMaybeZero>
__device__ __forceinline__ void mfma4_decode3(f32x16& c0, f32x16& c1, f32x16& c2, f32x16& c3, const f16x8& b,
                                              const f16x8 (&a)[4], uint32_t wx, uint32_t sx, uint32_t wy,
                                              uint32_t sy, uint32_t wz, uint32_t sz, f16x8& ox, f16x8& oy,
                                              f16x8& oz, uint32_t zero) {
  uint32_t x0, x1, x2, x3, y0, y1, y2, y3, z0, z1, z2, z3;
#define NVFP4_BODY3(OPS, MF)                                                                              \
  "s_nop 1\n\t" MF("c0") NVFP4_DEC_PAIR("x0", "wx", "sx", "", OPS)                                        \
      NVFP4_DEC_PAIR("x1", "wx", "sx", " op_sel:[1,0,0]", OPS)                                            \
      NVFP4_DEC_PAIR("x2", "wx", "sx", " op_sel:[0,1,0]", OPS) MF("c1")                                   \
      NVFP4_DEC_PAIR("x3", "wx", "sx", " op_sel:[1,1,0]", OPS) NVFP4_DEC_PAIR("y0", "wy", "sy", "", OPS)  \
      NVFP4_DEC_PAIR("y1", "wy", "sy", " op_sel:[1,0,0]", OPS) MF("c2")                                   \
      NVFP4_DEC_PAIR("y2", "wy", "sy", " op_sel:[0,1,0]", OPS)                                            \
      NVFP4_DEC_PAIR("y3", "wy", "sy", " op_sel:[1,1,0]", OPS) NVFP4_DEC_PAIR("z0", "wz", "sz", "", OPS)  \
      MF("c3") NVFP4_DEC_PAIR("z1", "wz", "sz", " op_sel:[1,0,0]", OPS)                                   \
      NVFP4_DEC_PAIR("z2", "wz", "sz", " op_sel:[0,1,0]", OPS) NVFP4_DEC_PAIR("z3", "wz", "sz", " op_sel:[1,1,0]", OPS)
#define NVFP4_OUT3                                                                                         \
  [c0] "+a"(c0), [c1] "+a"(c1), [c2] "+a"(c2), [c3] "+a"(c3), [x0] "=&v"(x0), [x1] "=&v"(x1), [x2] "=&v"(x2), \
      [x3] "=&v"(x3), [y0] "=&v"(y0), [y1] "=&v"(y1), [y2] "=&v"(y2), [y3] "=&v"(y3), [z0] "=&v"(z0),         \
      [z1] "=&v"(z1), [z2] "=&v"(z2), [z3] "=&v"(z3)
#define NVFP4_IN3                                                                                          \
  [b] "v"(b), [ac0] "v"(a[0]), [ac1] "v"(a[1]), [ac2] "v"(a[2]), [ac3] "v"(a[3]), [wx] "v"(wx), [sx] "v"(sx), \
      [wy] "v"(wy), [sy] "v"(sy), [wz] "v"(wz), [sz] "v"(sz)
  if constexpr (kHi && kMaybeZero)
    asm volatile(NVFP4_EITHER(NVFP4_BODY3(NVFP4_OPS_HI, NVFP4_MFMA_ZERO), NVFP4_BODY3(NVFP4_OPS_HI, NVFP4_MFMA_ACC))
                 : NVFP4_OUT3 : NVFP4_IN3, [z] "s"(zero) : "scc");
  else if constexpr (kHi)
    asm volatile(NVFP4_BODY3(NVFP4_OPS_HI, NVFP4_MFMA_ACC) : NVFP4_OUT3 : NVFP4_IN3);
  else if constexpr (kMaybeZero)
    asm volatile(NVFP4_EITHER(NVFP4_BODY3(NVFP4_OPS_LO, NVFP4_MFMA_ZERO), NVFP4_BODY3(NVFP4_OPS_LO, NVFP4_MFMA_ACC))
                 : NVFP4_OUT3 : NVFP4_IN3, [z] "s"(zero) : "scc");
  else
    asm volatile(NVFP4_BODY3(NVFP4_OPS_LO, NVFP4_MFMA_ACC) : NVFP4_OUT3 : NVFP4_IN3);
#undef NVFP4_BODY3
#undef NVFP4_OUT3
#undef NVFP4_IN3
  ox = __builtin_bit_cast(f16x8, u32x4{x0, x1, x2, x3});
  oy = __builtin_bit_cast(f16x8, u32x4{y0, y1, y2, y3});
  oz = __builtin_bit_cast(f16x8, u32x4{z0, z1, z2, z3});
}

// k16-step n of a stage read from LDS stage S: the codes and scales of
// sub-chunk s + 1 are read at step 4 s and converted at step 4 s + 2; the
// step's 4 FN MFMAs (operands decoded one step earlier) carry the decode of
// step n + 1, which for n = 15 is the first step of the next stage (its
// sub-chunk 0 is read in buffer 0 at step 12).  After the last stage of a
// workgroup that decode works on stale registers and is never used.  With
// FN = 4 blocks 0-1 decode the next step's A frags and blocks 2-3 its B
// frags; with FN = 3 block 2 decodes all three B frags.
template <int n, int FN, bool kMaybeZero = false>
__device__ __forceinline__ void fast_step(const FastStage<FN>& S, FastPipe<FN>& P, f32x16 (&acc)[FN][4],
                                          const FastLane& L, const FastRefill<FN>& rf, uint32_t zero = 0) {
  // copies of the refill after every kRefillEvery-th MFMA block from step kRefillStep on (3 or 4 blocks a step)
  constexpr int kBlocks = FN == 4 ? 4 : 3;
  constexpr int j0 = (n - kRefillStep) * kBlocks;  // MFMA block index from the first refill step
  constexpr int s = n >> 2, t = n & 3;
  if constexpr (t == 0 && s < 3) fast_read_sub(S, P, (s + 1) & 1, L, s + 1);
  if constexpr (t == 2 && s < 3) fast_convert_scales(P, (s + 1) & 1);
  if constexpr (n == 14) fast_convert_scales(P, 0);
  constexpr int c = n & 1, x = c ^ 1;
  // the next step: word t1 of the sub-chunk in buffer u1
  constexpr int t1 = (n + 1) & 3, u1 = n < 15 ? ((n + 1) >> 2) & 1 : 0;
  constexpr bool hi = t1 >= 2;
  const uint4* A = P.ca[u1];
  const uint4* B = P.cb[u1];
  mfma4_decode2<hi, kMaybeZero>(acc[0][0], acc[0][1], acc[0][2], acc[0][3], P.bv[c][0], P.av[c], word_of(A[0], t1), P.sa[u1][0],
                    word_of(A[1], t1), P.sa[u1][1], P.av[x][0], P.av[x][1], zero);
  if constexpr (n >= kRefillStep && (j0 + 0) % kRefillEvery == 0) rf.template copy<kRefillBurst + (j0 + 0) / kRefillEvery>();
  mfma4_decode2<hi, kMaybeZero>(acc[1][0], acc[1][1], acc[1][2], acc[1][3], P.bv[c][1], P.av[c], word_of(A[2], t1), P.sa[u1][2],
                    word_of(A[3], t1), P.sa[u1][3], P.av[x][2], P.av[x][3], zero);
  if constexpr (n >= kRefillStep && (j0 + 1) % kRefillEvery == 0) rf.template copy<kRefillBurst + (j0 + 1) / kRefillEvery>();
  if constexpr (FN == 4) {
    mfma4_decode2<hi, kMaybeZero>(acc[2][0], acc[2][1], acc[2][2], acc[2][3], P.bv[c][2], P.av[c], word_of(B[0], t1), P.sb[u1][0],
                      word_of(B[1], t1), P.sb[u1][1], P.bv[x][0], P.bv[x][1], zero);
    if constexpr (n >= kRefillStep && (j0 + 2) % kRefillEvery == 0) rf.template copy<kRefillBurst + (j0 + 2) / kRefillEvery>();
    mfma4_decode2<hi, kMaybeZero>(acc[3][0], acc[3][1], acc[3][2], acc[3][3], P.bv[c][3], P.av[c], word_of(B[2], t1), P.sb[u1][2],
                      word_of(B[3], t1), P.sb[u1][3], P.bv[x][2], P.bv[x][3], zero);
    if constexpr (n >= kRefillStep && (j0 + 3) % kRefillEvery == 0) rf.template copy<kRefillBurst + (j0 + 3) / kRefillEvery>();
  } else {
    static_assert(FN == 3, "FN is 3 or 4");
    mfma4_decode3<hi, kMaybeZero>(acc[2][0], acc[2][1], acc[2][2], acc[2][3], P.bv[c][2], P.av[c], word_of(B[0], t1), P.sb[u1][0],
                      word_of(B[1], t1), P.sb[u1][1], word_of(B[2], t1), P.sb[u1][2], P.bv[x][0], P.bv[x][1],
                      P.bv[x][2], zero);
    if constexpr (n >= kRefillStep && (j0 + 2) % kRefillEvery == 0) rf.template copy<kRefillBurst + (j0 + 2) / kRefillEvery>();
  }
}

static_assert(kBarrierStep >= 8 && kBarrierStep <= 11, "S is last read at step 8; Sn is first read at step 12");
static_assert(kRefillStep > kBarrierStep, "copies into S only after the barrier");

template <int n, int FN, bool kMaybeFirst>
__device__ __forceinline__ void fast_stage_steps(const FastStage<FN>& S, const FastStage<FN>& Sn, FastPipe<FN>& P,
                                                 f32x16 (&acc)[FN][4], const FastLane& L, const FastRefill<FN>& rf,
                                                 uint32_t first) {
  if constexpr (n < 16) {
    if constexpr (n == 12) fast_read_sub(Sn, P, 0, L, 0);
    fast_step<n, FN, kMaybeFirst && n == 0>(S, P, acc, L, rf, first);
    if constexpr (n == kBarrierStep) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      rf.whole_stage();
      rf.template burst<kRefillBurst>();
    }
    fast_stage_steps<n + 1, FN, kMaybeFirst>(S, Sn, P, acc, L, rf, first);
  }
}

// One stage (K = 256 = 4 sub-chunks x 4 k16-steps) from LDS stage S.  S is
// last read at step 8 (sub-chunk 3); after step kBarrierStep the waves
// synchronize (after which every copy into Sn has landed and nobody reads S
// any more), the copies of the stage after next into S (`rf`) are issued,
// part at once and the rest between the MFMA blocks of the following steps,
// and sub-chunk 0 of Sn is read at step 12 for the decode carried by step 15
// (after the last stage of a workgroup Sn holds stale data, read but never
// used).  In a tile's first stage (kMaybeFirst and `first` nonzero) the
// MFMAs of step 0 take a zero accumulator (an inline 0 as their C operand),
// which starts every output tile of the wave without writing 256 zeros to
// the accumulators first.
template <bool kMaybeFirst, int FN>
__device__ __forceinline__ void fast_stage(const FastStage<FN>& S, const FastStage<FN>& Sn, FastPipe<FN>& P,
                                           f32x16 (&acc)[FN][4], const FastLane& L, const FastRefill<FN>& rf,
                                           uint32_t first) {
  constexpr int kBlocks = FN == 4 ? 4 : 3;
  static_assert(kRefillBurst + (16 - kRefillStep) * kBlocks / kRefillEvery >= FastRefill<FN>::kCopies,
                "every copy of the refill is issued within the stage");
  fast_stage_steps<0, FN, kMaybeFirst>(S, Sn, P, acc, L, rf, first);
}

// Epilogue of one tile: lane (r, h), accumulator element e of MFMA tile (j, i)
// is output row m = 32 i + r and column n = 32 j + 8 (e / 4) + 4 h + e % 4;
// one 8-byte (bf16) or 16-byte (fp32) store per 4 consecutive columns.  All
// output stores are non-temporal: an output larger than the MALL gains
// nothing from being kept there (1.5-2% faster than plain stores).
// The accumulators of one MFMA tile, read out only where the epilogue uses
// them.  Without the empty asm the compiler reads all the accumulators into
// VGPRs ahead of the full/edge branch (both paths read them), runs out of
// VGPRs and spills; the reloads then wait, since vmcnt also counts stores,
// for every output store issued before them.
__device__ __forceinline__ f32x16 pinned(f32x16& acc) {
  f32x16 v;
#pragma unroll
  for (int e = 0; e < 16; e++) {
    float x;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(acc[e]));
    v[e] = x;
  }
  return v;
}

template <bool kBf16Out>
__device__ __forceinline__ void fast_store4(void* __restrict__ c, int64_t idx, const f32x16& a, int gq, float g) {
  const float v0 = a[4 * gq] * g, v1 = a[4 * gq + 1] * g, v2 = a[4 * gq + 2] * g, v3 = a[4 * gq + 3] * g;
  if constexpr (kBf16Out) {
    const bf16x2 p0 = {(__bf16)v0, (__bf16)v1}, p1 = {(__bf16)v2, (__bf16)v3};
    __builtin_nontemporal_store(u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)},
                                reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(c) + idx));
  } else {
    __builtin_nontemporal_store(f32x4{v0, v1, v2, v3}, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(c) + idx));
  }
}

// Tiles that cross row M or column N: every store checks its row and column.
template <bool kBf16Out, int FN>
__device__ __forceinline__ void fast_epilogue_edge(f32x16 (&acc)[FN][4], void* __restrict__ c, int64_t m0,
                                                   int64_t n0, int M, int N, int wm, int wn, int r, int h, float g) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t m = m0 + wm * 128 + 32 * i + r;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const f32x16 a = pinned(acc[j][i]);
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int64_t n = n0 + wn * 32 * FN + 32 * j + 8 * gq + 4 * h;
        if (n >= N) continue;  // N % 4 == 0: the 4 columns are all in or all out
        fast_store4<kBf16Out>(c, m * N + n, a, gq, g);
      }
    }
  }
}

// Two packed bf16 of a[4 gq + 2 e], a[4 gq + 2 e + 1] times g.
__device__ __forceinline__ uint32_t bf16_pair(const f32x16& a, int gq, int e, float g) {
  const bf16x2 p = {(__bf16)(a[4 * gq + 2 * e] * g), (__bf16)(a[4 * gq + 2 * e + 1] * g)};
  return __builtin_bit_cast(uint32_t, p);
}

// NJ (1 or 2) B frags j0 .. j0 + NJ - 1 of A frag i, bf16, staged through the
// wave-private 4 KiB LDS chunk `wl` (32 rows x 128 bytes, the 16-byte pieces
// of row r at slot ^ (r / 2) % 8, conflict-free both ways): lane (r, h) writes
// its 8-byte groups in the MFMA layout, then lanes read back 16 bytes each so
// that a store instruction covers 8 (NJ = 2: one whole 128-byte line per row)
// or 16 rows (NJ = 1: 64 contiguous bytes per row).  `dst0` is the output
// element of row 0, column 32 j0 of the run.
template <int NJ, int FN>
__device__ __forceinline__ void bf16_run(f32x16 (&acc)[FN][4], int i, int j0, __bf16* __restrict__ dst0,
                                         uint32_t N, int r, int h, float g, uint8_t* wl) {
  const int lane = threadIdx.x & 63;
  const uint32_t wsw = (uint32_t)((r >> 1) & 7);
  uint8_t* const wrow = wl + r * 128 + 8 * h;
#pragma unroll
  for (int jj = 0; jj < NJ; jj++) {
    const f32x16 a = pinned(acc[j0 + jj][i]);
#pragma unroll
    for (int gq = 0; gq < 4; gq++) {
      const uint32_t chunk = (uint32_t)(4 * jj + gq);
      *reinterpret_cast<u32x2*>(wrow + 16 * (chunk ^ wsw)) = u32x2{bf16_pair(a, gq, 0, g), bf16_pair(a, gq, 1, g)};
    }
  }
  constexpr int kLanesPerRow = 4 * NJ, kRowsPerStore = 64 / kLanesPerRow;
  const int rr0 = lane / kLanesPerRow, slot = lane % kLanesPerRow;
#pragma unroll
  for (int k = 0; k < 32 / kRowsPerStore; k++) {
    const int rr = rr0 + kRowsPerStore * k;
    const u32x4 v = *reinterpret_cast<const u32x4*>(wl + rr * 128 + 16 * (slot ^ ((rr >> 1) & 7)));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst0 + ((uint32_t)rr * N + 8u * (uint32_t)slot)));
  }
}

// Full tiles of an output with fewer than 2^32 elements, bf16, through the
// wave's LDS chunk so that the stores write whole 128-byte lines: pairs of
// adjacent B frags (64 columns, 128 bytes, 128-byte aligned since the tile's
// column offset is a multiple of 64).  With FN = 3 wave 0 covers columns
// 0-95 of the tile (frags 0-1 paired, frag 2 alone) and wave 1 columns 96-191
// (frag 0 alone, frags 1-2 paired): the two single frags share one line.
template <int FN>
__device__ __forceinline__ void fast_epilogue_full_bf16(f32x16 (&acc)[FN][4], void* __restrict__ c, int64_t m0,
                                                        int64_t n0, int N, int wm, int wn, int r, int h, float g,
                                                        uint8_t* wl) {
  const uint32_t row0 = (uint32_t)m0 + (uint32_t)(wm * 128), col0 = (uint32_t)n0 + (uint32_t)(wn * 32 * FN);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    __bf16* d = reinterpret_cast<__bf16*>(c) + ((row0 + 32u * i) * (uint32_t)N + col0);
    if constexpr (FN == 4) {
      bf16_run<2>(acc, i, 0, d, (uint32_t)N, r, h, g, wl);
      bf16_run<2>(acc, i, 2, d + 64, (uint32_t)N, r, h, g, wl);
    } else if (wn == 0) {
      bf16_run<2>(acc, i, 0, d, (uint32_t)N, r, h, g, wl);
      bf16_run<1>(acc, i, 2, d + 64, (uint32_t)N, r, h, g, wl);
    } else {
      bf16_run<1>(acc, i, 0, d, (uint32_t)N, r, h, g, wl);
      bf16_run<2>(acc, i, 1, d + 32, (uint32_t)N, r, h, g, wl);
    }
  }
}

// Full tiles, fp32 output: 16-byte stores straight from the MFMA layout.
template <int FN>
__device__ __forceinline__ void fast_epilogue_full_f32(f32x16 (&acc)[FN][4], void* __restrict__ c, int64_t m0,
                                                       int64_t n0, int N, int wm, int wn, int r, int h, float g) {
  const uint32_t row0 = (uint32_t)m0 + (uint32_t)(wm * 128 + r);
  const uint32_t col0 = (uint32_t)n0 + (uint32_t)(wn * 32 * FN + 4 * h);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float* row = reinterpret_cast<float*>(c) + ((row0 + 32u * i) * (uint32_t)N + col0);
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const f32x16 a = pinned(acc[j][i]);
#pragma unroll
      for (int gq = 0; gq < 4; gq++) fast_store4<false>(row + 32 * j + 8 * gq, 0, a, gq, g);
    }
  }
}

// Persistent fast-path kernel: one workgroup per CU walks tiles lin, lin + G,
// lin + 2G, ... (G = grid size).  Workgroups are dealt round-robin to the 8
// XCDs, so lin is remapped to keep the tiles processed concurrently by one
// XCD contiguous (they then share A and B rows in that XCD's L2).  Stages
// stream through the two LDS stages across tile boundaries: the copies of
// the next tile's first two stages are issued during the current tile's last
// two, and the epilogue stores are not waited for, so neither the store
// drain, the tile turnover nor the first fetch stalls the matrix cores.
// Tiles are 256 x 64 FN.
template <bool kBf16Out, int FN>
__global__ __launch_bounds__(256, 1) void gemm_w4a4_fast_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_sg,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, const float* __restrict__ b_sg, int M,
    int N, int K, void* __restrict__ c, int tiles_m, int tiles_n) {
  constexpr int kTN = 64 * FN;  // B rows (output columns) per tile
  __shared__ FastStage<FN> st0;
  __shared__ FastStage<FN> st1;
  __shared__ __attribute__((aligned(16))) uint8_t epi[4][4096];  // per-wave output staging (bf16)
  const int T = tiles_m * tiles_n;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int lin0 = (G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;
  const int nk = K / kFastKC;  // even, >= 2
  const float g = a_sg[0] * b_sg[0];
  const bool small_c = (int64_t)M * N < (int64_t(1) << 32);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar branches on wn
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5;

  const FastLoad ld = fast_load_offsets(K);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)&st0);
  const uint32_t lds1 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)&st1);
  int tm, tn;
  tile_of_lin(lin0, tiles_m, tiles_n, tm, tn);
  bool edge = (int64_t)(tm + 1) * kTile > M || (int64_t)(tn + 1) * kTN > N;
  fast_load_stage<FN>(lds0, ld, edge, a_codes, a_scales, b_codes, b_scales, (int64_t)tm * kTile, (int64_t)tn * kTN,
                      M, N, K, 0);
  fast_load_stage<FN>(lds1, ld, edge, a_codes, a_scales, b_codes, b_scales, (int64_t)tm * kTile, (int64_t)tn * kTN,
                      M, N, K, 1);
  // Wait for stage 0 only: stage 1 is first read at step 12 of stage 0, after
  // that stage's barrier, which waits for every copy.  Loads complete in
  // order, and stage 1's copies are this wave's last 8 + 2 FN + 1 (or one
  // more), so at most that many outstanding means stage 0 has landed.
  // s_waitcnt fields (gfx9): vmcnt bits 3:0 and 15:14, expcnt 6:4 and
  // lgkmcnt 11:8 left at their maxima.
  constexpr int kStage1Copies = 8 + 2 * FN + 1;
  __builtin_amdgcn_s_waitcnt((kStage1Copies & 15) | ((kStage1Copies >> 4) << 14) | (7 << 4) | (15 << 8));
  __syncthreads();
  FastLane L;
  L.a = (uint32_t)(wm * 128 + r) * 128;
  L.b = (uint32_t)(wn * 32 * FN + r) * 128;
  L.sa = (uint32_t)(wm * 128 + r) * 16 + 2 * h;
  L.sb = (uint32_t)(wn * 32 * FN + r) * 16 + 2 * h;
  L.hsw = 16u * (uint32_t)(h ^ ((r >> 1) & 7));
  FastPipe<FN> P;

  for (int lin = lin0; lin < T; lin += G) {
    // First k16-step of the tile, from stage 0 in st0.  Decoding it here
    // rather than in the previous tile's last step keeps the pipeline
    // registers dead across the epilogue, which then has the VGPRs it needs
    // (spill reloads there would wait for all of the tile's output stores).
    fast_read_sub(st0, P, 0, L, 0);
    fast_convert_scales(P, 0);
    fast_decode_first(P);
    const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTN;
    const bool has_next = lin + G < T;
    int tm_next = tm, tn_next = tn;
    if (has_next) tile_of_lin(lin + G, tiles_m, tiles_n, tm_next, tn_next);
    const bool edge_next = (int64_t)(tm_next + 1) * kTile > M || (int64_t)(tn_next + 1) * kTN > N;
    const int64_t m0_next = (int64_t)tm_next * kTile, n0_next = (int64_t)tn_next * kTN;
    // Not zeroed: the first k16-step of the tile writes every accumulator
    // with zero-C MFMAs (nk >= 2, so every tile runs that step).  The empty
    // asm statements give them a defined value without any instruction (left
    // undefined, the register allocator spills around the tile loop).
    f32x16 acc[FN][4];
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) asm volatile("" : "=a"(acc[j][i]));
    for (int kc = 0; kc < nk; kc += 2) {
      // stage kc (st0), then kc + 1 (st1); each refills its LDS stage with
      // the stage two later: kc + 2 of this tile or, at the end of the tile,
      // stage 0 / 1 of the next tile.
      const bool more = kc + 2 < nk;
      // the stage two later: kc + 2 / kc + 3 of this tile, or stage 0 / 1 of the next
      const int64_t rm0 = more ? m0 : m0_next, rn0 = more ? n0 : n0_next;
      const bool redge = more ? edge : edge_next, ron = more || has_next;
      const int rkc = more ? kc + 2 : 0;
      fast_stage<true>(st0, st1, P, acc, L,
                       FastRefill<FN>(lds0, ld, ron, redge, a_codes, a_scales, b_codes, b_scales, rm0, rn0, M, N, K, rkc),
                       __builtin_amdgcn_readfirstlane(kc == 0 ? 1u : 0u));
      fast_stage<false>(st1, st0, P, acc, L,
                        FastRefill<FN>(lds1, ld, ron, redge, a_codes, a_scales, b_codes, b_scales, rm0, rn0, M, N, K,
                                       rkc + 1),
                        0u);
    }
    // The stores drain while the next tile computes (the next wait comes
    // 12 k16-steps later).
    if (!edge && small_c) {
      if constexpr (kBf16Out)
        fast_epilogue_full_bf16(acc, c, m0, n0, N, wm, wn, r, h, g, epi[wave]);
      else
        fast_epilogue_full_f32(acc, c, m0, n0, N, wm, wn, r, h, g);
    } else
      fast_epilogue_edge<kBf16Out>(acc, c, m0, n0, M, N, wm, wn, r, h, g);
    tm = tm_next;
    tn = tn_next;
    edge = edge_next;
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_sg, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_sg, int64_t M, int64_t N, int64_t K, void* c,
                       int c_dtype, hipStream_t stream) {
  constexpr int WM = NVFP4_GEMM_WM, WN = NVFP4_GEMM_WN;
  const int tiles_m = (int)((M + kTile - 1) / kTile), tiles_n = (int)((N + kTile - 1) / kTile);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
  const bool fast = (K % kKC == 0) && ((uintptr_t)a_codes % 16 == 0) && ((uintptr_t)b_codes % 16 == 0) &&
                    ((uintptr_t)a_scales % 8 == 0) && ((uintptr_t)b_scales % 8 == 0);
  const bool bf = c_dtype == kDtypeBf16;
  const bool dma = K > 0 && (K % (2 * kFastKC) == 0) && (N % 4 == 0) && (M * (K / 2) < (int64_t(1) << 32)) &&
                   (N * (K / 2) < (int64_t(1) << 32)) && ((uintptr_t)a_codes % 16 == 0) &&
                   ((uintptr_t)b_codes % 16 == 0) && ((uintptr_t)a_scales % 16 == 0) &&
                   ((uintptr_t)b_scales % 16 == 0) && ((uintptr_t)c % 16 == 0);
  if (dma) {
    // 256 x 256 tiles, or 256 x 192 ones when those take fewer rounds of the
    // persistent grid, a round of the smaller tiles counting as kCost192 of a
    // full one: they hold 3/4 of the MFMA work, but the copies, barriers and
    // epilogue per tile shrink less (measured 0.81-0.93 on 2048-8192 x 3072 x
    // 3072).  4096 x 3072 outputs: 192 tiles of 256 x 256 leave a quarter of
    // 256 CUs idle; 256 tiles of 256 x 192 fill them.
    constexpr double kCost192 = 0.87;
    const int cus = device_cu_count();
    const int64_t tn192 = (N + 191) / 192;
    const int64_t rounds256 = ((int64_t)tiles_m * tiles_n + cus - 1) / cus;
    const int64_t rounds192 = ((int64_t)tiles_m * tn192 + cus - 1) / cus;
    const bool t192 = (double)rounds192 * kCost192 < (double)rounds256;
    const int tn = t192 ? (int)tn192 : tiles_n;
    const int T = tiles_m * tn;
    const dim3 pgrid((unsigned)(T < cus ? T : cus));
#define NVFP4_FAST_LAUNCH(B, FN)                                                                                  \
  launch_kernel(gemm_w4a4_fast_kernel<B, FN>, pgrid, dim3(256), 0, stream, a_codes, a_scales, a_sg, b_codes, b_scales, \
                b_sg, (int)M, (int)N, (int)K, c, tiles_m, tn)
    if (t192) return bf ? NVFP4_FAST_LAUNCH(true, 3) : NVFP4_FAST_LAUNCH(false, 3);
    return bf ? NVFP4_FAST_LAUNCH(true, 4) : NVFP4_FAST_LAUNCH(false, 4);
#undef NVFP4_FAST_LAUNCH
  }
#define NVFP4_GEMM_LAUNCH(F, B)                                                                      \
  launch_kernel(gemm_w4a4_kernel<WM, WN, F, B>, grid, block, 0, stream, a_codes, a_scales, a_sg, b_codes, \
                b_scales, b_sg, (int)M, (int)N, (int)K, c, tiles_m, tiles_n)
  if (fast) return bf ? NVFP4_GEMM_LAUNCH(true, true) : NVFP4_GEMM_LAUNCH(true, false);
  return bf ? NVFP4_GEMM_LAUNCH(false, true) : NVFP4_GEMM_LAUNCH(false, false);
#undef NVFP4_GEMM_LAUNCH
}

}  // namespace nvfp4
