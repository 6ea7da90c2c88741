// Softmax attention of bf16 queries over an NVFP4 KV cache, for gfx950.
//
// The LongLive-2.0 pages restore the NVFP4 KV cache with a parallel
// dequantization kernel for the attention (d9249.github.io review, "Core idea /
// structure / operation"; arXiv abstract: the KV cache is held in NVFP4).
// Here the attention reads the packed cache directly: each 64-token block of
// K and V is decoded once per workgroup into LDS, exactly (a decoded element
// val(q) * val(s) has at most 6 significant bits: exact in bf16 and fp16),
// so HBM only carries the 0.5625 B/element of the packed cache.
//
//   o[h][i][:] = s_gV[h] * sum_j w_j v_j / sum_j w_j,
//   w_j = exp(scale * s_gK[h] * (q_i . k_j) - max),  k_j, v_j without s_g.
//
// Per workgroup: 256 queries of one head (8 waves x 32, one MFMA column tile
// each; two waves per SIMD, so one wave's softmax overlaps the other's
// MFMAs).  Per block:
//   S^T = K . Q^T   v_mfma_f32_32x32x16_bf16 (bf16 queries, exact bf16 K;
//                   products exact in fp32), so each lane holds the scores of
//                   ONE query (16 of a 32-token tile; the other 16 sit in lane
//                   l ^ 32): the row maximum needs one cross-half exchange;
//   online softmax  exp2 of scores pre-multiplied by scale * s_gK * log2(e),
//                   a lazily updated running max m (moved only when a block
//                   exceeds it by 2^8) and per-lane partial sums l in fp32;
//   O^T += V^T P^T  v_mfma_f32_32x32x16_f16 (P rounded to fp16, exact fp16
//                   V).  The A operand needs 8 consecutive tokens of one
//                   head-dim column per lane while the cache is token-major:
//                   two ds_read_b64_tr_b16 (transposing LDS reads) per operand
//                   deliver them from V stored [token][d] in LDS.
// The tokens of an MFMA k-step are ordered to match the score layout, so P
// goes from the softmax to the MFMA without any exchange.
//
// Load balance (flash-decoding split): when (query blocks x heads) would
// leave CUs idle or a ragged last round, the cache is cut into `splits`
// ranges of whole blocks, one workgroup per (query block, head, range); each
// writes its unnormalised O, running max m and sum l in fp32 to a workspace
// and a combine kernel merges the ranges:
//   o = s_gV * sum_r 2^(m_r - M) O_r / sum_r 2^(m_r - M) l_r,  M = max_r m_r.
//
// LDS layouts (64 tokens x 256 B each, swizzled so that the decode writes,
// the K operand reads and the transposing V reads are all bank-conflict
// free):
//   K  [token][16 slots of 16 B] bf16, chunk c (d = 8c..8c+7) in slot
//      c ^ (token % 16);
//   V  [token][32 slots of 8 B] fp16, chunk c (d = 4c..4c+3) in slot
//      c ^ (8 (token % 4) + 2 ((token / 4) % 4)).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/nvfp4.h"
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

// Scratch of kv_attention_noalloc, for callers that cannot allocate: the
// split-cache partial results (fp32 O, m, l per range and query) live in this
// fixed array instead of a caller workspace.  Each device the library runs on
// holds its own copy until the process ends.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __fp16 fp16x4_raw __attribute__((__vector_size__(8)));  // operand type of the transposing read
typedef __attribute__((address_space(3))) fp16x4_raw lds_fp16x4;

constexpr int kAD = 128;         // head_dim
constexpr int kABN = 64;         // cache tokens per block
constexpr int kAQW = 32;         // queries per wave
constexpr int kAW = 8;           // waves per workgroup
constexpr int kABM = kAW * kAQW; // queries per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;  // log2 of the largest probability before the maximum moves

struct AttnSmem {
  uint8_t k[kABN * 256];
  uint8_t v[kABN * 256];
};

// Packed codes and scale byte of one token and one NVFP4 block of head_dim
// (d = 16 qd .. 16 qd + 15) of K and of V: thread tid takes token tid % 64 of
// the cache block and qd = tid / 64.
struct RawKV {
  u32x2 kc, vc;
  uint32_t ks, vs;
};

__device__ __forceinline__ void load_raw(RawKV& r, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
                                         const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs, int64_t tok,
                                         int qd) {
  r.kc = *reinterpret_cast<const u32x2*>(kc + tok * (kAD / 2) + 8 * qd);
  r.vc = *reinterpret_cast<const u32x2*>(vc + tok * (kAD / 2) + 8 * qd);
  r.ks = ks[tok * (kAD / 16) + qd];
  r.vs = vs[tok * (kAD / 16) + qd];
}

// Codes of byte P of w times the block scale: two exact bf16 (K) or fp16 (V).
template <int P>
__device__ __forceinline__ uint32_t k_pair(uint32_t w, float sv) {
  const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, P);
  const bf16x2 b = {(__bf16)(f.x * sv), (__bf16)(f.y * sv)};
  return __builtin_bit_cast(uint32_t, b);
}
template <int P>
__device__ __forceinline__ uint32_t v_pair(uint32_t w, f16x2 sv) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, P) * sv);
}

// Decode the thread's 16 K and 16 V elements into LDS (exact bf16 / fp16).
__device__ __forceinline__ void decode_to_lds(const RawKV& r, AttnSmem& sm, int t, int qd) {
  const float ksv = e4m3_value(r.ks);
  const f16x2 vsv = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs | (r.vs << 8), 1.0f, false);
#pragma unroll
  for (int wi = 0; wi < 2; wi++) {  // 8 elements d = 16 qd + 8 wi + (0..7)
    const uint32_t kw = wi ? r.kc.y : r.kc.x;
    const uint32_t kp[4] = {k_pair<0>(kw, ksv), k_pair<1>(kw, ksv), k_pair<2>(kw, ksv), k_pair<3>(kw, ksv)};
    const int kslot = (2 * qd + wi) ^ (t & 15);
    *reinterpret_cast<u32x4*>(sm.k + t * 256 + kslot * 16) = u32x4{kp[0], kp[1], kp[2], kp[3]};

    const uint32_t vw = wi ? r.vc.y : r.vc.x;
    const uint32_t vp[4] = {v_pair<0>(vw, vsv), v_pair<1>(vw, vsv), v_pair<2>(vw, vsv), v_pair<3>(vw, vsv)};
    const int vslot = (4 * qd + 2 * wi) ^ (8 * (t & 3) + 2 * ((t >> 2) & 3));  // even: two adjacent 8-B slots
    *reinterpret_cast<u32x4*>(sm.v + t * 256 + vslot * 8) = u32x4{vp[0], vp[1], vp[2], vp[3]};
  }
}

// A operand of S^T = K . Q^T for token tile tau, k-step s: this lane's token
// 32 tau + lane % 32, head-dim 16 s + 8 (lane / 32) .. + 7.
__device__ __forceinline__ bf16x8 k_frag(const AttnSmem& sm, int tau, int s, int lane) {
  const int tok = 32 * tau + (lane & 31);
  const int slot = (2 * s + (lane >> 5)) ^ (tok & 15);
  return *reinterpret_cast<const bf16x8*>(sm.k + tok * 256 + slot * 16);
}

// A operand of O^T = V^T . P^T for head-dim tile dt and k-step (tau, nu):
// lane l gets head-dim 32 dt + l % 32 and the 8 tokens of k = 8 (l / 32) + i,
// token(i) = 32 tau + 16 nu + 8 (i / 4) + 4 (l / 32) + i % 4 (the order in
// which the score layout holds them).  Each of the two transposing reads
// covers i = 4c .. 4c + 3: within a group of 16 lanes, lane i gets element
// i % 4 of the 8-byte chunks addressed by lanes i / 4 + 4 j (j = 0..3), so
// lane s of the group addresses token(4c + s / 4), head-dim chunk
// 8 dt + 4 ((l / 16) % 2) + s % 4.
__device__ __forceinline__ f16x8 v_frag(const AttnSmem& sm, int dt, int tau, int nu, int lane) {
  const int hh = lane >> 5, g = (lane >> 4) & 1, s16 = lane & 15;
  const int q = s16 & 3, j = s16 >> 2;
  f16x4 part[2];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int tok = 32 * tau + 16 * nu + 8 * c + 4 * hh + j;
    const int chunk = 8 * dt + 4 * g + q;
    const int slot = chunk ^ (8 * j + 2 * ((2 * c + hh) & 3));  // tok % 4 == j, (tok / 4) % 4 == (2c + hh) % 4
    part[c] = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                            (lds_fp16x4*)((__attribute__((address_space(3))) uint8_t*)sm.v +
                                                          tok * 256 + slot * 8)));
  }
  return f16x8{part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
}

// Online softmax of one query tile for one block: scores s (2 token tiles x
// 16 per lane), running max m (log2 units) and sum l; returns the fp16
// probabilities as the B operands of the 4 k-steps of O^T += V^T P^T and the
// rescale factor of O.  Tokens from `valid` on lie past the end of the cache:
// their LDS rows repeat the last cached token, so they cannot move the
// maximum, and their probabilities are zeroed (only in a ragged last block)
// before the row sum, which is taken over the fp16 probabilities (v_dot2),
// the same values the second product uses.
__device__ __forceinline__ float softmax_tile(const f32x16 (&s)[2], float c, int valid, int hh, float& m, float& l,
                                              f16x8 (&pf)[4]) {
  // block maximum of c * s (c >= 0: a negative factor is folded into the
  // queries); the two halves of the wave exchange theirs with one lane swap
  float bm = s[0][0];
#pragma unroll
  for (int i = 1; i < 32; i++) bm = fmaxf(bm, s[i >> 4][i & 15]);
  bm *= c;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  // Lazy maximum: the reference point only moves when the block maximum
  // exceeds it by more than 2^8, so probabilities stay <= 256 (fp16 keeps its
  // 2^-11 relative rounding there) and the output rescale is rare.
  const float m_new = bm > m + kLazyLog2 ? bm : m;
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  m = m_new;
#pragma unroll
  for (int u = 0; u < 4; u++) {  // k-step u: token tile u / 2, elements 8 (u % 2) .. + 7
    const f32x16& st = s[u >> 1];
    _Float16 p[8];
#pragma unroll
    for (int i = 0; i < 8; i++) p[i] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(st[8 * (u & 1) + i], c, -m_new));
    pf[u] = f16x8{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
  }
  if (valid < kABN) {
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int e = 8 * (u & 1) + i;
        const int tok = 32 * (u >> 1) + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (tok >= valid) pf[u][i] = (_Float16)0.0f;
      }
  }
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int i = 0; i < 4; i++)
      sum = __builtin_amdgcn_fdot2(f16x2{pf[u][2 * i], pf[u][2 * i + 1]}, f16x2{(_Float16)1.0f, (_Float16)1.0f}, sum,
                                   false);
  l = l * alpha + sum;
  return alpha;
}

// One cache block (in LDS) against the wave's 32 queries: S^T = K . Q^T,
// online softmax, O^T += V^T . P^T.
__device__ __forceinline__ void attn_block(const AttnSmem& cur, const bf16x8 (&qf)[8], f32x16 (&oacc)[4], float& m,
                                           float& l, float c_k, int valid, int lane) {
  // S^T = K . Q^T: sacc[tau], lane (query n, half hh), element e ->
  // token 32 tau + 8 (e / 4) + 4 hh + e % 4.
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
  {
    // K operands read two k-steps ahead of their MFMAs
    bf16x8 kf[3];
    kf[0] = k_frag(cur, 0, 0, lane);
    kf[1] = k_frag(cur, 0, 1, lane);
#pragma unroll
    for (int st = 0; st < 16; st++) {
      if (st + 2 < 16) kf[(st + 2) % 3] = k_frag(cur, (st + 2) >> 3, (st + 2) & 7, lane);
      sacc[st >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st % 3], qf[st & 7], sacc[st >> 3], 0, 0, 0);
    }
  }

  f16x8 pf[4];
  const float alpha = softmax_tile(sacc, c_k, valid, lane >> 5, m, l, pf);
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {  // the running max moved for some query
#pragma unroll
    for (int dt = 0; dt < 4; dt++) oacc[dt] *= alpha;
  }
  // O^T += V^T . P^T, operands read one k-step ahead of their MFMAs.
  f16x8 vf[2];
  vf[0] = v_frag(cur, 0, 0, 0, lane);
#pragma unroll
  for (int st = 0; st < 16; st++) {
    if (st + 1 < 16) vf[(st + 1) & 1] = v_frag(cur, (st + 1) >> 2, ((st + 1) & 3) >> 1, (st + 1) & 1, lane);
    oacc[st >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[st & 1], pf[st & 3], oacc[st >> 2], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kAW * 64, 1) void attn_nvfp4_kv_kernel(
    const __bf16* __restrict__ q, const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const float* __restrict__ k_hs, const uint8_t* __restrict__ v_codes, const uint8_t* __restrict__ v_scales,
    const float* __restrict__ v_hs, int q_tokens, int64_t cache_tokens, int kv_tokens, float scale,
    __bf16* __restrict__ out, int blocks_per_split, float* __restrict__ part_o, float2* __restrict__ part_ml) {
  __shared__ AttnSmem sm[2];
  const int h = blockIdx.y;
  // this workgroup's cache blocks [blk0, blk1) (never empty: the host sizes the ranges)
  const int blk0 = blockIdx.z * blocks_per_split;
  const int blk1 = min((kv_tokens + kABN - 1) / kABN, blk0 + blocks_per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int64_t cache_row0 = (int64_t)h * cache_tokens;
  const uint8_t* kc = k_codes + cache_row0 * (kAD / 2);
  const uint8_t* ks = k_scales + cache_row0 * (kAD / 16);
  const uint8_t* vc = v_codes + cache_row0 * (kAD / 2);
  const uint8_t* vs = v_scales + cache_row0 * (kAD / 16);
  const float c_raw = scale * k_hs[h] * kLog2e;  // raw dot product -> log2 units
  // a negative factor is folded into the queries (exact bf16 negation)
  const float c_k = __builtin_fabsf(c_raw);
  const uint32_t qsign = c_raw < 0.0f ? 0x80008000u : 0u;
  const float s_gv = v_hs[h];

  // Queries of this wave (one column tile of 32); rows past q_tokens repeat the last row.
  const int qbase = blockIdx.x * kABM + wave * kAQW;
  bf16x8 qf[8];
  {
    const int qi = min(qbase + n, q_tokens - 1);
    const __bf16* qrow = q + ((int64_t)h * q_tokens + qi) * kAD;
#pragma unroll
    for (int s = 0; s < 8; s++) {
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hh) ^ qsign);
      // opaque from here on: otherwise the compiler re-loads the queries
      // from memory in every block and the first MFMAs wait for them
      asm volatile("" : "+v"(qf[s]));
    }
  }

  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m = -INFINITY, l = 0.0f;

  // First block decoded into sm[0], the next prefetched into registers.
  const int t_dec = threadIdx.x & 63, qd_dec = threadIdx.x >> 6;  // token, NVFP4 block of head_dim
  RawKV raw;
  load_raw(raw, kc, ks, vc, vs, min(blk0 * kABN + t_dec, kv_tokens - 1), qd_dec);
  decode_to_lds(raw, sm[0], t_dec, qd_dec);
  if (blk0 + 1 < blk1) load_raw(raw, kc, ks, vc, vs, min((blk0 + 1) * kABN + t_dec, kv_tokens - 1), qd_dec);
  __syncthreads();

  // One block from `cur`; then the next block is decoded into `nxt` (its last
  // readers finished before the previous barrier) and the one after is
  // prefetched.  Unrolled by two so that each buffer is a compile-time LDS
  // offset (the operand reads then need no per-block address arithmetic).
  auto step = [&](int blk, AttnSmem& cur, AttnSmem& nxt) {
    attn_block(cur, qf, oacc, m, l, c_k, kv_tokens - blk * kABN, lane);
    if (blk + 1 < blk1) {
      decode_to_lds(raw, nxt, t_dec, qd_dec);
      if (blk + 2 < blk1) load_raw(raw, kc, ks, vc, vs, min((blk + 2) * kABN + t_dec, kv_tokens - 1), qd_dec);
    }
    __syncthreads();
  };
  for (int blk = blk0; blk < blk1; blk += 2) {
    step(blk, sm[0], sm[1]);
    if (blk + 1 < blk1) step(blk + 1, sm[1], sm[0]);
  }

  // l = this lane's partial sum + the other half's.
  const float lt = l + __shfl_xor(l, 32);
  const int qi = qbase + n;
  if (part_o) {  // one range of a split cache: unnormalised O, m, l for the combine
    if (qi < q_tokens) {
      const int64_t row = ((int64_t)blockIdx.z * gridDim.y + h) * q_tokens + qi;
      float* prow = part_o + row * kAD;
#pragma unroll
      for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int eg = 0; eg < 4; eg++) {
          const f32x16& a = oacc[dt];
          *reinterpret_cast<f32x4*>(prow + 32 * dt + 8 * eg + 4 * hh) =
              f32x4{a[4 * eg], a[4 * eg + 1], a[4 * eg + 2], a[4 * eg + 3]};
        }
      if (hh == 0) part_ml[row] = make_float2(m, lt);
    }
    return;
  }
  // o = s_gV * O / l
  const float inv = s_gv / lt;
  if (qi < q_tokens) {
    __bf16* orow = out + ((int64_t)h * q_tokens + qi) * kAD;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int eg = 0; eg < 4; eg++) {  // head-dim 32 dt + 8 eg + 4 hh + (0..3)
        const f32x16& a = oacc[dt];
        const bf16x2 p0 = {(__bf16)(a[4 * eg] * inv), (__bf16)(a[4 * eg + 1] * inv)};
        const bf16x2 p1 = {(__bf16)(a[4 * eg + 2] * inv), (__bf16)(a[4 * eg + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * eg + 4 * hh) =
            u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
      }
  }
}

// Merge the cache ranges of a split attention: 32 lanes per query, 4 head-dim
// columns each.
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           const float* __restrict__ v_hs, int splits, int heads,
                                                           int q_tokens, __bf16* __restrict__ out) {
  const int64_t rows = (int64_t)heads * q_tokens;
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
  if (row >= rows) return;
  const int c4 = (threadIdx.x & 31) * 4;
  float mx = -INFINITY;
  for (int r = 0; r < splits; r++) mx = fmaxf(mx, part_ml[r * rows + row].x);
  float lsum = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r = 0; r < splits; r++) {
    const float2 ml = part_ml[r * rows + row];
    const float w = __builtin_amdgcn_exp2f(ml.x - mx);
    lsum = __builtin_fmaf(w, ml.y, lsum);
    const f32x4 o = *reinterpret_cast<const f32x4*>(part_o + (r * rows + row) * kAD + c4);
    acc += w * o;
  }
  const float inv = v_hs[row / q_tokens] / lsum;
  const bf16x2 p0 = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
  const bf16x2 p1 = {(__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)};
  *reinterpret_cast<u32x2*>(out + row * kAD + c4) = u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
}

struct AttnSplit {
  int splits;            // cache ranges (1: no split, no workspace)
  int blocks_per_split;  // cache blocks per range
};

int64_t split_workspace_bytes(int64_t heads, int64_t q_tokens, int splits) {
  return splits > 1 ? (int64_t)splits * heads * q_tokens * (kAD * 4 + 8) : 0;
}

// The number of cache ranges that minimises the modelled time, in units of one
// workgroup's pass over one cache block: rounds of resident workgroups (one
// per CU) x (blocks per range + a fixed start-up cost), plus the partial
// results' HBM round trip in the combine.  Only splits whose workspace fits in
// max_bytes are considered.
AttnSplit choose_split(int64_t heads, int64_t q_tokens, int64_t kv_tokens, int64_t max_bytes) {
  const int64_t wgs = (q_tokens + kABM - 1) / kABM * heads;
  const int64_t nblk = (kv_tokens + kABN - 1) / kABN;
  const int64_t cus = device_cu_count();
  AttnSplit best{1, (int)nblk};
  double best_cost = 0.0;
  for (int sp = 1; sp <= 32; sp++) {
    const int64_t bps = (nblk + sp - 1) / sp;
    if ((nblk + bps - 1) / bps != sp || (sp > 1 && bps < 4)) continue;  // every range non-empty, >= 4 blocks
    if (split_workspace_bytes(heads, q_tokens, sp) > max_bytes) continue;
    const double rounds = (double)((wgs * sp + cus - 1) / cus);
    double cost = rounds * (double)(bps + 3);
    if (sp > 1) cost += 3.0 + (double)(split_workspace_bytes(heads, q_tokens, sp) + heads * q_tokens * kAD * 2) / 5.2e6;
    if (sp == 1 || cost < best_cost) {
      best_cost = cost;
      best = AttnSplit{sp, (int)bps};
    }
  }
  return best;
}

}  // namespace

int64_t kv_attention_workspace_bytes(int64_t heads, int64_t q_tokens, int64_t kv_tokens) {
  if (q_tokens == 0) return 0;
  const AttnSplit sp = choose_split(heads, q_tokens, kv_tokens, INT64_MAX);
  return split_workspace_bytes(heads, q_tokens, sp.splits);
}

hipError_t launch_kv_attention(const void* q, const uint8_t* k_codes, const uint8_t* k_scales, const float* k_hs,
                               const uint8_t* v_codes, const uint8_t* v_scales, const float* v_hs, int64_t heads,
                               int64_t q_tokens, int64_t cache_tokens, int64_t kv_tokens, float scale, void* out,
                               void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (q_tokens == 0) return hipSuccess;
  const AttnSplit sp = choose_split(heads, q_tokens, kv_tokens, workspace ? workspace_bytes : 0);
  const dim3 grid((unsigned)((q_tokens + kABM - 1) / kABM), (unsigned)heads, (unsigned)sp.splits);
  float* part_o = sp.splits > 1 ? static_cast<float*>(workspace) : nullptr;
  float2* part_ml = sp.splits > 1 ? reinterpret_cast<float2*>(part_o + (int64_t)sp.splits * heads * q_tokens * kAD)
                                  : nullptr;
  hipError_t e = launch_kernel(attn_nvfp4_kv_kernel, grid, dim3(kAW * 64), 0, stream, (const __bf16*)q, k_codes,
                               k_scales, k_hs, v_codes, v_scales, v_hs, (int)q_tokens, cache_tokens, (int)kv_tokens,
                               scale, (__bf16*)out, sp.blocks_per_split, part_o, part_ml);
  if (e != hipSuccess || sp.splits == 1) return e;
  const int64_t threads = heads * q_tokens * 32;
  return launch_kernel(attn_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       (const float*)part_o, (const float2*)part_ml, v_hs, sp.splits, (int)heads, (int)q_tokens,
                       (__bf16*)out);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up with that device current on the
// first call for it.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_kv_attention_noalloc(const void* q, const uint8_t* k_codes, const uint8_t* k_scales,
                                       const float* k_hs, const uint8_t* v_codes, const uint8_t* v_scales,
                                       const float* v_hs, int64_t heads, int64_t q_tokens, int64_t cache_tokens,
                                       int64_t kv_tokens, float scale, void* out, hipStream_t stream) {
  if (q_tokens == 0) return hipSuccess;
  void* ws = nullptr;
  const hipError_t e = scratch_address(stream, &ws);
  if (e != hipSuccess) return e;
  // The same kernels as kv_attention with a workspace of the scratch's size:
  // no split whose partial results would not fit is chosen, so every size
  // kv_attention accepts runs (one pass needs no scratch at all).
  return launch_kv_attention(q, k_codes, k_scales, k_hs, v_codes, v_scales, v_hs, heads, q_tokens, cache_tokens,
                             kv_tokens, scale, out, ws, (int64_t)NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}

}  // namespace nvfp4
