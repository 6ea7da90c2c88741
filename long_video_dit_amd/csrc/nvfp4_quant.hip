// NVFP4 quantize / dequantize kernels for gfx950 (MI355X).
//
// Layout: a tensor is processed as G equal groups (G = 1 for a plain
// tensor, G = heads for the KV cache), each group a flat run of elements
// with its own fp32 scale.  Inside a group the work unit of one lane is 8
// consecutive elements (16 B of bf16, 32 B of fp32); in the amax pass lanes
// 2j and 2j+1 share one 16-element block, and an encode lane owns two units,
// a whole block.  All kernels are HBM-bound grid-stride loops; the encode
// and dequantize passes go in chunks (a lane's loads of a pass issued
// together and waited for once, then its stores), because loads and stores
// share one wait counter.
//
//   amax_partial_kernel  pass 1: per-block max |x| -> partials (fp32 bits)
//   finalize_kernel      per group: max of partials -> s_g = RN(amax / 2688)
//   amax_slot_kernel     standalone s_g: atomic max into the s_g slot itself
//   encode_kernel        pass 2: scale byte and 16 codes per block, a block
//                        per lane (optionally FourOverSix: the better of two
//                        candidate scales per block)
//   encode_t_kernel      pass 2 along the other axis: NVFP4 of x^T
//   dequant_kernel       codes + scales -> bf16 / fp32, 8 outputs per lane
//
// The amax partials live in the caller's codes buffer (it is at least 4 B
// per 8 elements), which the encode pass overwrites afterwards; the calls
// therefore need no workspace and no atomics, and the scale is deterministic.
#include <hip/hip_runtime.h>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int kThreads = 256;

// ---- element loads: 8 consecutive elements as fp32 -----------------------

__device__ __forceinline__ void load8(const uint16_t* __restrict__ x, int64_t unit, float (&f)[8]) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + unit);
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ void load8(const float* __restrict__ x, int64_t unit, float (&f)[8]) {
  const f32x4* p = reinterpret_cast<const f32x4*>(x) + 2 * unit;
  const f32x4 a = __builtin_nontemporal_load(p);
  const f32x4 b = __builtin_nontemporal_load(p + 1);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// max |x| of 8 elements as non-negative fp32 bits (integer order = float order)
__device__ __forceinline__ uint32_t amax8_bits(const uint16_t* __restrict__ x, int64_t unit) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + unit);
  uint32_t m = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    m = __builtin_elementwise_max(m, w[i] & 0x7fffu);
    m = __builtin_elementwise_max(m, (w[i] >> 16) & 0x7fffu);
  }
  return m << 16;
}

__device__ __forceinline__ uint32_t amax8_bits(const float* __restrict__ x, int64_t unit) {
  float f[8];
  load8(x, unit, f);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) m = __builtin_elementwise_max(m, __float_as_uint(f[i]) & 0x7fffffffu);
  return m;
}

template <int kNT = kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* smem) {
  // wavefront reduction, then across the kNT / 64 waves of the block
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_elementwise_max(v, (uint32_t)__shfl_xor((int)v, off));
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) smem[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kNT / 64; i++) v = __builtin_elementwise_max(v, smem[i]);
  }
  return v;
}

// grid: (P, G).  Block b of group g reduces units b*? grid-stride and writes
// partials[g * P + b].
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const T* __restrict__ x, int64_t units_per_group,
                                                                uint32_t* __restrict__ partials) {
  __shared__ uint32_t smem[kThreads / 64];
  const int g = blockIdx.y;
  const T* xg = x + (int64_t)g * units_per_group * 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m = 0;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + 3 * stride < units_per_group; u += 4 * stride) {
    const uint32_t a = amax8_bits(xg, u), b = amax8_bits(xg, u + stride);
    const uint32_t c = amax8_bits(xg, u + 2 * stride), d = amax8_bits(xg, u + 3 * stride);
    m = __builtin_elementwise_max(m, __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                               __builtin_elementwise_max(c, d)));
  }
  for (; u < units_per_group; u += stride) m = __builtin_elementwise_max(m, amax8_bits(xg, u));
  m = block_max_u32(m, smem);
  if (threadIdx.x == 0) partials[(int64_t)g * gridDim.x + blockIdx.x] = m;
}

// grid: G blocks of kFinThreads.  s_g[g] = RN_f32(max(partials of g) / 2688).
// A thread issues its (up to 4) loads of a pass before reducing them, so up
// to 4096 partials cost one memory round trip rather than one per partial.
constexpr int kFinThreads = 1024;

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(const uint32_t* __restrict__ partials, int P,
                                                               float* __restrict__ s_g) {
  __shared__ uint32_t smem[kFinThreads / 64];
  const int g = blockIdx.x;
  const uint32_t* pg = partials + (int64_t)g * P;
  uint32_t m = 0;
  for (int i0 = 0; i0 < P; i0 += 4 * kFinThreads) {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = i0 + j * kFinThreads + (int)threadIdx.x;
      v[j] = i < P ? pg[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) m = __builtin_elementwise_max(m, v[j]);
  }
  m = block_max_u32<kFinThreads>(m, smem);
  if (threadIdx.x == 0) {
    // IEEE division is correctly rounded: one RNE of amax / 2688.
    s_g[g] = __fdiv_rn(__uint_as_float(m), 2688.0f);
  }
}

// ---- standalone per-tensor scale: the s_g slot is the reduction target ----

// slot <- 0 (a kernel rather than a memset node, so the call can be captured).
__global__ void zero_slot_kernel(uint32_t* __restrict__ slot) { slot[0] = 0u; }

// Every workgroup folds the max |x| bits of its units into the slot with one
// atomic max (order-free, so the result does not depend on scheduling).
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_slot_kernel(const T* __restrict__ x, int64_t units,
                                                             uint32_t* __restrict__ slot) {
  __shared__ uint32_t smem[kThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m = 0;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + 3 * stride < units; u += 4 * stride) {
    const uint32_t a = amax8_bits(x, u), b = amax8_bits(x, u + stride);
    const uint32_t c = amax8_bits(x, u + 2 * stride), d = amax8_bits(x, u + 3 * stride);
    m = __builtin_elementwise_max(m, __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                               __builtin_elementwise_max(c, d)));
  }
  for (; u < units; u += stride) m = __builtin_elementwise_max(m, amax8_bits(x, u));
  m = block_max_u32(m, smem);
  if (threadIdx.x == 0) atomicMax(slot, m);
}

// slot (max |x| as fp32 bits) -> s_g = RN(amax / 2688), in place.
__global__ void finalize_slot_kernel(float* __restrict__ s_g) {
  s_g[0] = __fdiv_rn(__uint_as_float(reinterpret_cast<const uint32_t*>(s_g)[0]), 2688.0f);
}

// One 8-element unit as loaded (16 B of bf16 or 32 B of fp32), converted to
// fp32 only when it is encoded, so that the next units' loads can be issued
// first.  Non-temporal loads: plain ones were ~4% faster with the tensor
// already in the caches, but ~25% slower after other data had filled the MALL
// (its dirty lines are then written back during the read).
template <typename T>
struct Raw8;

template <>
struct Raw8<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* __restrict__ x, int64_t unit) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + unit);
  }
  __device__ __forceinline__ void unpack(float (&f)[8]) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* __restrict__ x, int64_t unit) {
    const f32x4* p = reinterpret_cast<const f32x4*>(x) + 2 * unit;
    a = __builtin_nontemporal_load(p);
    b = __builtin_nontemporal_load(p + 1);
  }
  __device__ __forceinline__ void unpack(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// The scale byte and the two code words of one 16-element block: the usual
// encoding, or with k46 (FourOverSix) the one of the two candidate scales that
// dequantizes with the smaller squared error.  Returns false when k46 and the
// fast comparison cannot decide (a near-tie): the caller settles the block
// with encode_block_settle, outside its loop (that path calls functions, and
// a call inside the encode loops makes the compiler spill to scratch on every
// block).
template <bool k46>
__device__ __forceinline__ bool encode_block(const float (&f0)[8], const float (&f1)[8], float am,
                                             const EncodeConsts& c, uint32_t& sb, uint32_t& w0, uint32_t& w1) {
  sb = encode_scale(am, c);
  w0 = encode8(f0, sb, c);
  w1 = encode8(f1, sb, c);
  if constexpr (k46) {
    const uint32_t sb4 = encode_scale4(am, c);
    if (sb4 != sb) {
      const uint32_t x0 = encode8(f0, sb4, c), x1 = encode8(f1, sb4, c);
      const int d = prefer4_fast(f0, f1, w0, w1, sb, x0, x1, sb4, c);
      if (d < 0) return false;
      if (d == 1) {
        sb = sb4;
        w0 = x0;
        w1 = x1;
      }
    }
  }
  return true;
}

// FourOverSix encoding of one block with the decision always settled (the
// fp64 and exact comparisons after the fast one).
__device__ __noinline__ void encode_block_settle(const float (&f0)[8], const float (&f1)[8], float s_g,
                                                 uint32_t& sb, uint32_t& w0, uint32_t& w1) {
  const EncodeConsts c = make_encode_consts(s_g);  // built here: a reference would put it in scratch
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(f0[i]), __builtin_fabsf(f1[i])));
  sb = encode_scale(am, c);
  w0 = encode8(f0, sb, c);
  w1 = encode8(f1, sb, c);
  const uint32_t sb4 = encode_scale4(am, c);
  if (sb4 != sb) {
    const uint32_t x0 = encode8(f0, sb4, c), x1 = encode8(f1, sb4, c);
    if (prefer4(f0, f1, w0, w1, sb, x0, x1, sb4, c)) {
      sb = sb4;
      w0 = x0;
      w1 = x1;
    }
  }
}

// Blocks of a workgroup whose FourOverSix decision is left to after its
// encode loop: entries (iteration << 8 | thread), at most 4 per thread (the
// launcher sizes the grid for that).
constexpr int kPendMax = 4 * kThreads;

// The grid-stride loop of one lane over whole 16-element blocks b0,
// b0 + stride, ... < nb of one group (units 2b and 2b + 1), used by the
// FourOverSix mode (its arithmetic, not memory, bounds it; the chunked loop
// below was no faster there).  The block maximum needs no lane exchange and a
// lane stores 8 B of codes and its block's scale byte.  The loads of the next
// block are issued before the current one is encoded; their indexes are
// clamped to the last block (always in bounds) and the stores need no
// predicate.
template <typename T, bool k46>
__device__ __forceinline__ void encode_lane_blocks(const T* __restrict__ xg, int64_t nb, int64_t b0, int64_t stride,
                                                   const EncodeConsts& c, uint32_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, int64_t base, uint32_t* pend,
                                                   uint32_t* npend) {
  const int64_t last = nb - 1;
  Raw8<T> nxt[2];
  {
    const int64_t bb = __builtin_elementwise_min(b0, last);
    nxt[0].load(xg, 2 * bb);
    nxt[1].load(xg, 2 * bb + 1);
  }
  uint32_t it = 0;
  for (int64_t bk = b0; bk < nb; bk += stride, it++) {
    const Raw8<T> cur[2] = {nxt[0], nxt[1]};
    const int64_t bn = __builtin_elementwise_min(bk + stride, last);
    nxt[0].load(xg, 2 * bn);
    nxt[1].load(xg, 2 * bn + 1);
    float f0[8], f1[8];
    cur[0].unpack(f0);
    cur[1].unpack(f1);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(f0[i]), __builtin_fabsf(f1[i])));
    uint32_t sb, w0, w1;
    if (!encode_block<k46>(f0, f1, am, c, sb, w0, w1)) {
      pend[atomicAdd(npend, 1u)] = (it << 8) | threadIdx.x;
      continue;
    }
    __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(codes + base) + bk);
    scales[(base >> 1) + bk] = (uint8_t)sb;
  }
}

// Blocks per lane per pass of encode_lane_chunks: 2 bf16 blocks or 1 fp32
// block, 64 bytes and 16 VGPRs of loads (88 VGPRs in all, 5 waves per SIMD).
// Measured on bf16 tensors of 12.6M-235M elements and the KV cache: 1 or 2
// blocks per lane are equal, 3 are 5% slower, 4 (120 VGPRs, 4 waves) 3-5%
// slower and 8 30% slower.
template <typename T>
struct EncodeChunk {
  static constexpr int kBlocks = sizeof(T) == 2 ? 2 : 1;
};

// The plain (not FourOverSix) encode of whole 16-element blocks, in passes:
// pass p of workgroup w takes chunk ch = w + p * gridDim.x, whose lane t
// encodes blocks ch * kBlocks * kThreads + j * kThreads + t (j < kBlocks).  A
// pass issues all of its loads, waits for them once, then encodes and stores
// every block.  gfx950 counts loads and stores on one counter, and the
// compiler cannot wait for a load issued after a store without waiting for
// the store too: a loop that loads the next block while storing the current
// one waits each iteration for its stores to land.  Here a pass waits once,
// for its loads and the previous pass's stores together.  Loads past the last
// block are clamped to it (in bounds) and their stores skipped.
template <typename T>
struct EncodeChunkRegs {
  Raw8<T> r[EncodeChunk<T>::kBlocks][2];

  __device__ __forceinline__ void load(const T* __restrict__ xg, int64_t ch, int64_t last) {
#pragma unroll
    for (int j = 0; j < EncodeChunk<T>::kBlocks; j++) {
      const int64_t bk =
          __builtin_elementwise_min(ch * EncodeChunk<T>::kBlocks * kThreads + j * kThreads + threadIdx.x, last);
      r[j][0].load(xg, 2 * bk);
      r[j][1].load(xg, 2 * bk + 1);
    }
  }

  __device__ __forceinline__ void encode(int64_t ch, int64_t nb, const EncodeConsts& c, uint32_t* __restrict__ codes,
                                         uint8_t* __restrict__ scales, int64_t base) const {
#pragma unroll
    for (int j = 0; j < EncodeChunk<T>::kBlocks; j++) {
      const int64_t bk = ch * EncodeChunk<T>::kBlocks * kThreads + j * kThreads + threadIdx.x;
      float f0[8], f1[8];
      r[j][0].unpack(f0);
      r[j][1].unpack(f1);
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++)
        am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(f0[i]), __builtin_fabsf(f1[i])));
      uint32_t sb, w0, w1;
      encode_block<false>(f0, f1, am, c, sb, w0, w1);
      if (bk < nb) {
        __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(codes + base) + bk);
        scales[(base >> 1) + bk] = (uint8_t)sb;
      }
    }
  }
};

// The passes from the workgroup's second on; the first chunk is already in
// flight in `rg`.
template <typename T>
__device__ __forceinline__ void encode_lane_chunks(EncodeChunkRegs<T>& rg, const T* __restrict__ xg, int64_t nb,
                                                   const EncodeConsts& c, uint32_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, int64_t base) {
  constexpr int64_t kSpan = (int64_t)EncodeChunk<T>::kBlocks * kThreads;
  for (int64_t ch = blockIdx.x;;) {
    __builtin_amdgcn_s_waitcnt(0);
    rg.encode(ch, nb, c, codes, scales, base);
    ch += gridDim.x;
    if (ch * kSpan >= nb) break;
    rg.load(xg, ch, nb - 1);
  }
}

// The loop with the encoder's mode read at run time (a tiny or zero s_g), as
// a function of its own for FourOverSix: its calls need registers saved across
// them, and inside the kernel the compiler would hoist those scratch stores
// ahead of the usual-mode loop as well.
template <typename T, bool k46>
__device__ __noinline__ void encode_lane_blocks_any_mode(const T* __restrict__ xg, int64_t nb, int64_t b0,
                                                         int64_t stride, float s_g, uint32_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t base, uint32_t* pend,
                                                         uint32_t* npend) {
  const EncodeConsts c = make_encode_consts(s_g);  // built here: a reference would put it in scratch
  encode_lane_blocks<T, k46>(xg, nb, b0, stride, c, codes, scales, base, pend, npend);
}

// grid: (X, G).  Each lane encodes whole 16-element blocks.  Group g reads
// units [g * units_per_group, (g + 1) * units_per_group) of x and writes them
// at unit g * out_group_stride + out_offset of the codes (and the matching
// scale bytes): a plain tensor has out_group_stride = units_per_group and
// out_offset = 0; a KV-cache append writes a slice of each head's rows.  Both
// are even (whole blocks), so the 8-byte code stores stay aligned.  The
// common case (an ordinary per-tensor scale) runs a copy of the loop in which
// the encoder's mode is the constant 0, so that no mode test is left inside.
// k46: FourOverSix block scaling; the workgroup settles its undecided blocks
// after the loop.
template <typename T, bool k46>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(k46 ? 4 : 1, 8))) void encode_kernel(
    const T* __restrict__ x, int64_t units_per_group,
                                                          const float* __restrict__ s_g,
                                                          uint32_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int64_t out_group_stride,
                                                          int64_t out_offset) {
  __shared__ uint32_t pend[k46 ? kPendMax : 1];
  __shared__ uint32_t npend;
  if (k46) {
    if (threadIdx.x == 0) npend = 0;
    __syncthreads();
  }
  const int g = blockIdx.y;
  const int64_t base = (int64_t)g * out_group_stride + out_offset;
  const T* xg = x + (int64_t)g * units_per_group * 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t b0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nb = units_per_group / 2;
  // The plain encode issues its first chunk's loads before it reads s_g and
  // builds the constants (two dependent scalar loads and fp64 divisions).
  // The grid never exceeds the chunk count, so every workgroup has one.
  EncodeChunkRegs<T> rg;
  if constexpr (!k46) rg.load(xg, blockIdx.x, nb - 1);
  const EncodeConsts c = make_encode_consts(s_g[g]);
  if constexpr (!k46) {
    if (c.mode == 0) {
      EncodeConsts cf = c;
      cf.mode = 0;
      encode_lane_chunks<T>(rg, xg, nb, cf, codes, scales, base);
    } else {
      encode_lane_chunks<T>(rg, xg, nb, c, codes, scales, base);
    }
  } else if (c.mode == 0) {
    EncodeConsts cf = c;
    cf.mode = 0;
    encode_lane_blocks<T, k46>(xg, nb, b0, stride, cf, codes, scales, base, pend, &npend);
  } else {
    encode_lane_blocks_any_mode<T, k46>(xg, nb, b0, stride, c.s_g, codes, scales, base, pend, &npend);
  }
  if constexpr (k46) {
    __syncthreads();
    const uint32_t n = npend;
    for (uint32_t e = threadIdx.x; e < n; e += kThreads) {
      const uint32_t ent = pend[e];
      const int64_t bk = (int64_t)blockIdx.x * kThreads + (ent & 0xffu) + (int64_t)(ent >> 8) * stride;
      Raw8<T> r0, r1;
      r0.load(xg, 2 * bk);
      r1.load(xg, 2 * bk + 1);
      float f0[8], f1[8];
      r0.unpack(f0);
      r1.unpack(f1);
      uint32_t sb, w0, w1;
      encode_block_settle(f0, f1, c.s_g, sb, w0, w1);
      __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(codes + base) + bk);
      scales[(base >> 1) + bk] = (uint8_t)sb;
    }
  }
}

// val(code) of the two nibbles of byte S of w, times the block scale (exact).
template <int S>
__device__ __forceinline__ void decode_pair(uint32_t w, float sv, float* p) {
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, S);
  p[0] = d.x * sv;
  p[1] = d.y * sv;
}

// Units per lane per pass of the dequantizer (see dequant_kernel).
constexpr int kDequantChunk = 2;

// grid: (X, G).  One lane per 8-element unit (4 code bytes, the block's scale
// byte) -> 8 outputs, so that every store instruction of a wave writes one
// contiguous span (1 KiB of bf16).  Splitting a lane's output over two
// strided 16-byte stores instead costs ~30% extra HBM write traffic.  A lane
// takes kDequantChunk units per pass (units ch * kDequantChunk * kThreads +
// j * kThreads + lane), loads them all, waits once and then decodes and
// stores them: loads and stores share one wait counter, so a loop that loads
// while earlier stores are in flight waits for those stores as well (one unit
// per iteration was 8-14% slower).  Loads past the end are clamped (in
// bounds) and their stores skipped.
template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           int64_t units_per_group, const float* __restrict__ s_g,
                                                           void* __restrict__ y) {
  const int g = blockIdx.y;
  const float sg = s_g[g];
  const int64_t base = (int64_t)g * units_per_group;
  const int64_t last = units_per_group - 1;
  constexpr int64_t kSpan = (int64_t)kDequantChunk * kThreads;
  for (int64_t ch = blockIdx.x; ch * kSpan < units_per_group; ch += gridDim.x) {
    uint32_t wv[kDequantChunk], sbv[kDequantChunk];
#pragma unroll
    for (int j = 0; j < kDequantChunk; j++) {
      const int64_t u = __builtin_elementwise_min(ch * kSpan + j * kThreads + threadIdx.x, last);
      wv[j] = __builtin_nontemporal_load(codes + base + u);
      sbv[j] = scales[(base + u) >> 1];
    }
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int j = 0; j < kDequantChunk; j++) {
      const int64_t u = ch * kSpan + j * kThreads + threadIdx.x;
      if (u > last) break;
      const uint32_t w = wv[j];
      const float sv = e4m3_value(sbv[j]);
      float p[8];  // val(code) * val(scale), exact: <= 6 significant bits
      decode_pair<0>(w, sv, p + 0);
      decode_pair<1>(w, sv, p + 2);
      decode_pair<2>(w, sv, p + 4);
      decode_pair<3>(w, sv, p + 6);
      if constexpr (kBf16Out) {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; i++) o[i] = bf16_of_product(p[2 * i], sg) | (bf16_of_product(p[2 * i + 1], sg) << 16);
        __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4*>(y) + (base + u));
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(y) + 2 * (base + u);
        __builtin_nontemporal_store(f32x4{p[0] * sg, p[1] * sg, p[2] * sg, p[3] * sg}, dst);
        __builtin_nontemporal_store(f32x4{p[4] * sg, p[5] * sg, p[6] * sg, p[7] * sg}, dst + 1);
      }
    }
  }
}

// ---- transposed encode ---------------------------------------------------
//
// x [rows][cols] -> the NVFP4 form of x^T: codes [cols][rows / 2], scales
// [cols][rows / 16], blocks of 16 consecutive rows of one column (the layout
// the backward GEMMs contract over: dgrad over the output features of W,
// wgrad over tokens).  One 512-thread workgroup per tile of 256 rows x 128
// columns; lane
// (c4 = lane % 16 + 16 (wave / 4), rb = 4 (wave % 4) + lane / 16) owns
// columns 4 c4 .. 4 c4 + 3 and rows 16 rb .. 16 rb + 15 of the tile, i.e.
// four whole blocks, so the block maximum needs no lane exchange.  Loads: the
// 16 lanes of one rb read 128 contiguous bytes of bf16, and a tile reads
// 256-byte row segments.  Codes and scale bytes are staged
// in LDS per tile and stored column by column, 16 lanes x 8 B = one 128-byte
// line of codes per column and 16 scale bytes per column, instead of 32-byte
// pieces of 16 columns per instruction.  Same rounding helpers as the
// row-wise pass, so the result is bit-identical to quantizing x^T.
constexpr int kTR = 256, kTC = 128, kTThreads = 512;

template <typename T>
__device__ __forceinline__ void load4(const T* __restrict__ p, float (&f)[4]);
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* __restrict__ p, float (&f)[4]) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4<float>(const float* __restrict__ p, float (&f)[4]) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  f[0] = v.x;
  f[1] = v.y;
  f[2] = v.z;
  f[3] = v.w;
}
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

template <typename T, bool kVec, bool k46>
__global__ __launch_bounds__(kTThreads) void encode_t_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                            const float* __restrict__ s_g,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  // Staging: codes [kTC = 128 columns][32 words + 2 pad], scales [128 columns][16 B].
  __shared__ uint32_t sc[kTC][34];
  __shared__ uint32_t ss[kTC][4];
  __shared__ uint32_t pend[k46 ? 4 * kTThreads : 1];  // (column j << 9 | thread) of undecided FourOverSix blocks
  __shared__ uint32_t npend;
  if (k46) {
    if (threadIdx.x == 0) npend = 0;
    __syncthreads();
  }
  const EncodeConsts c = make_encode_consts(s_g[0]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Tile order: workgroup ids go round-robin over the 8 XCDs.  When row and
  // column tiles both come in eights, XCD x takes the column tiles = x (mod 8)
  // of one group of 8 row tiles at a time: the 8 row tiles that write one
  // 128-byte line of a column's scale bytes (16 bytes each) then run together
  // on one XCD, whose L2 merges them, and the tiles in flight cover 8 row
  // tiles by all columns.  On dY [16384, 14336] (same process): 216 us against
  // 222 us for row-major order, and 226 us when each XCD walked all the row
  // tiles of a column tile (accesses spread over every row at once).
  const int64_t tiles_c = (cols + kTC - 1) / kTC, tiles_r = (rows + kTR - 1) / kTR;
  int64_t tile_r, tile_c;
  if (tiles_c % 8 == 0 && tiles_r % 8 == 0) {
    const int64_t s8 = blockIdx.x / 8, rem = s8 % tiles_c;
    tile_r = 8 * (s8 / tiles_c) + rem % 8;
    tile_c = 8 * (rem / 8) + blockIdx.x % 8;
  } else {
    tile_r = blockIdx.x / tiles_c;
    tile_c = blockIdx.x % tiles_c;
  }
  const int64_t tr0 = tile_r * kTR, tc0 = tile_c * kTC;
  const int rb = 4 * (wave & 3) + (lane >> 4), c4 = (lane & 15) + 16 * (wave >> 2);
  const int64_t r0 = tr0 + 16 * rb, col0 = tc0 + 4 * c4;
  if (r0 < rows && col0 < cols) {  // rows % 16 == 0: a block is wholly in or out
    float f[4][16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const T* row = x + (r0 + i) * cols + col0;
      float v[4];
      if (kVec) {
        load4<T>(row, v);
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++) v[j] = col0 + j < cols ? load1(row + j) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; j++) f[j][i] = v[j];
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; i++) am = __builtin_fmaxf(am, __builtin_fabsf(f[j][i]));
      float lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo[i] = f[j][i];
        hi[i] = f[j][8 + i];
      }
      uint32_t sb, w0, w1;
      if (!encode_block<k46>(lo, hi, am, c, sb, w0, w1)) pend[atomicAdd(&npend, 1u)] = ((uint32_t)j << 9) | threadIdx.x;
      *reinterpret_cast<u32x2*>(&sc[4 * c4 + j][2 * rb]) = u32x2{w0, w1};
      reinterpret_cast<uint8_t*>(ss[4 * c4 + j])[rb] = (uint8_t)sb;
    }
  }
  __syncthreads();
  if constexpr (k46) {  // settle the undecided blocks in the staging buffers
    const uint32_t n = npend;
    for (uint32_t e = threadIdx.x; e < n; e += kTThreads) {
      const uint32_t ent = pend[e], t = ent & 511u, j = ent >> 9;
      const int ln = (int)(t & 63u), wv = (int)(t >> 6);
      const int rbe = 4 * (wv & 3) + (ln >> 4), c4e = (ln & 15) + 16 * (wv >> 2);
      const T* col = x + (tr0 + 16 * rbe) * cols + tc0 + 4 * c4e + j;
      float lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo[i] = load1(col + i * cols);
        hi[i] = load1(col + (8 + i) * cols);
      }
      uint32_t sb, w0, w1;
      encode_block_settle(lo, hi, c.s_g, sb, w0, w1);
      *reinterpret_cast<u32x2*>(&sc[4 * c4e + j][2 * rbe]) = u32x2{w0, w1};
      reinterpret_cast<uint8_t*>(ss[4 * c4e + j])[rbe] = (uint8_t)sb;
    }
    __syncthreads();
  }
  // Codes: 16 lanes per column, lane p stores rows 16 p .. 16 p + 15 (8 B),
  // non-temporal like the tile's loads (x is streamed once; the codes are
  // whole 128-byte lines).
  const int64_t words_per_col = rows / 8;
#pragma unroll
  for (int it = 0; it < kTC * 16 / kTThreads; it++) {
    const int idx = it * kTThreads + threadIdx.x, cl = idx >> 4, p = idx & 15;
    if (tc0 + cl < cols && tr0 + 16 * p < rows)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x2*>(&sc[cl][2 * p]),
                                  reinterpret_cast<u32x2*>(codes + (tc0 + cl) * words_per_col + tr0 / 8 + 2 * p));
  }
  // Scale bytes: 4 lanes per column, 4 bytes each when aligned.
  {
    static_assert(kTC * 4 == kTThreads, "one scale word per thread");
    const int cl = threadIdx.x >> 2, p = threadIdx.x & 3;
    if (tc0 + cl < cols) {
      uint8_t* dst = scales + (tc0 + cl) * (rows / 16) + tr0 / 16 + 4 * p;
      if (rows % 64 == 0 && tr0 + 64 * (p + 1) <= rows) {
        *reinterpret_cast<uint32_t*>(dst) = ss[cl][p];
      } else {
        for (int b = 0; b < 4; b++)
          if (tr0 + 16 * (4 * p + b) < rows) dst[b] = reinterpret_cast<const uint8_t*>(ss[cl])[4 * p + b];
      }
    }
  }
}

// ---- launchers ----------------------------------------------------------

static int grid_blocks(int64_t work_items, int per_thread, int max_blocks) {
  int64_t b = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (b < 1) b = 1;
  if (b > max_blocks) b = max_blocks;
  return (int)b;
}

hipError_t launch_global_scale(const void* x, int dtype, int64_t units_per_group, int groups, uint32_t* partials,
                               int64_t partial_capacity, float* s_g, hipStream_t stream) {
  const int cus = device_cu_count();
  // A tensor with one scale is read as `sub` equal slices, each with its own
  // partials, and finalized as one group.  Each workgroup then walks a slice
  // of a few tens of MB, so its in-flight loads lie ~1 MB apart instead of
  // ~16 MB: the activation [16384, 14336] reads at ~6.2 TB/s instead of
  // ~5.5 (the same layout as the per-head KV scales).
  int sub = 1;
  if (groups == 1) {
    for (int c : {32, 24, 16, 8})
      if (units_per_group % c == 0 && units_per_group / c >= (int64_t)1 << 18) {
        sub = c;
        break;
      }
  }
  const int64_t upg = units_per_group / sub;
  const int64_t slices = (int64_t)groups * sub;
  // Partials per slice: enough blocks to saturate HBM, bounded by the scratch.
  int64_t P = grid_blocks(upg, 8, (int)std::max<int64_t>(1, (int64_t)cus * 16 / slices));
  if (P * slices > partial_capacity) P = std::max<int64_t>(1, partial_capacity / slices);
  if (upg == 0) {
    P = 0;
  } else {
    const dim3 grid((unsigned)P, (unsigned)slices);
    hipError_t e;
    if (dtype == kDtypeF32)
      e = launch_kernel(amax_partial_kernel<float>, grid, dim3(kThreads), 0, stream, (const float*)x, upg, partials);
    else
      e = launch_kernel(amax_partial_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, (const uint16_t*)x, upg,
                        partials);
    if (e != hipSuccess) return e;
  }
  // group g's partials are slices g * sub .. g * sub + sub - 1: P * sub in a row
  return launch_kernel(finalize_kernel, dim3((unsigned)groups), dim3(kFinThreads), 0, stream, (const uint32_t*)partials,
                       (int)(P * sub), s_g);
}

hipError_t launch_finalize(const uint32_t* partials, int P, float* s_g, hipStream_t stream) {
  return launch_kernel(finalize_kernel, dim3(1), dim3(kFinThreads), 0, stream, partials, P, s_g);
}

hipError_t launch_global_scale_slot(const void* x, int dtype, int64_t units, float* s_g, hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(s_g);
  hipError_t e = launch_kernel(zero_slot_kernel, dim3(1), dim3(1), 0, stream, slot);
  if (e != hipSuccess) return e;
  if (units > 0) {
    const dim3 grid((unsigned)grid_blocks(units, 8, device_cu_count() * 16));
    if (dtype == kDtypeF32)
      e = launch_kernel(amax_slot_kernel<float>, grid, dim3(kThreads), 0, stream, (const float*)x, units, slot);
    else
      e = launch_kernel(amax_slot_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, (const uint16_t*)x, units, slot);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(finalize_slot_kernel, dim3(1), dim3(1), 0, stream, s_g);
}

hipError_t launch_encode(const void* x, int dtype, int64_t units_per_group, int groups, const float* s_g,
                         uint32_t* codes, uint8_t* scales, hipStream_t stream, int64_t out_group_stride,
                         int64_t out_offset, bool four_over_six) {
  if (units_per_group == 0) return hipSuccess;
  if (out_group_stride < 0) out_group_stride = units_per_group;
  // whole blocks: the kernel stores 8 bytes of codes per block
  if ((units_per_group | out_group_stride | out_offset) & 1) return hipErrorInvalidValue;
  const int cus = device_cu_count();
  int64_t bx;
  if (four_over_six) {
    // about three blocks per thread, up to 64 workgroups per CU, and at most
    // 4 blocks per thread, so a workgroup's undecided blocks always fit its
    // list (kPendMax)
    bx = grid_blocks(units_per_group, 6, std::max(1, cus * 64 / groups));
    bx = std::max<int64_t>(bx, (units_per_group / 2 + kPendMax - 1) / kPendMax);
  } else {
    // one chunk of EncodeChunk blocks per thread, up to 64 workgroups per CU
    const int kb = dtype == kDtypeF32 ? EncodeChunk<float>::kBlocks : EncodeChunk<uint16_t>::kBlocks;
    bx = grid_blocks(units_per_group, 2 * kb, std::max(1, cus * 64 / groups));
  }
  const dim3 grid((unsigned)bx, (unsigned)groups);
  auto go = [&](auto kernel, const auto* xt) {
    return launch_kernel(kernel, grid, dim3(kThreads), 0, stream, xt, units_per_group, s_g, codes, scales,
                         out_group_stride, out_offset);
  };
  if (dtype == kDtypeF32)
    return four_over_six ? go(encode_kernel<float, true>, (const float*)x) : go(encode_kernel<float, false>, (const float*)x);
  return four_over_six ? go(encode_kernel<uint16_t, true>, (const uint16_t*)x)
                       : go(encode_kernel<uint16_t, false>, (const uint16_t*)x);
}

hipError_t launch_encode_t(const void* x, int dtype, int64_t rows, int64_t cols, const float* s_g, uint32_t* codes,
                           uint8_t* scales, hipStream_t stream, bool four_over_six) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t tiles = (rows + kTR - 1) / kTR * ((cols + kTC - 1) / kTC);
  const dim3 grid((unsigned)tiles);
  const bool vec = cols % 4 == 0;
  auto go = [&](auto kernel, const auto* xt) {
    return launch_kernel(kernel, grid, dim3(kTThreads), 0, stream, xt, rows, cols, s_g, codes, scales);
  };
  const float* xf = (const float*)x;
  const uint16_t* xb = (const uint16_t*)x;
  if (dtype == kDtypeF32) {
    if (four_over_six) return vec ? go(encode_t_kernel<float, true, true>, xf) : go(encode_t_kernel<float, false, true>, xf);
    return vec ? go(encode_t_kernel<float, true, false>, xf) : go(encode_t_kernel<float, false, false>, xf);
  }
  if (four_over_six)
    return vec ? go(encode_t_kernel<uint16_t, true, true>, xb) : go(encode_t_kernel<uint16_t, false, true>, xb);
  return vec ? go(encode_t_kernel<uint16_t, true, false>, xb) : go(encode_t_kernel<uint16_t, false, false>, xb);
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* s_g, int64_t blocks_per_group,
                          int groups, void* y, int y_dtype, hipStream_t stream) {
  if (blocks_per_group == 0) return hipSuccess;
  const int64_t units = 2 * blocks_per_group;
  const int cus = device_cu_count();
  // one chunk per thread, up to 128 workgroups per CU (with one unit per
  // iteration: 92 against 105 us on one KV tensor with 16 per CU)
  const int bx = grid_blocks(units, kDequantChunk, std::max(1, cus * 128 / groups));
  const dim3 grid((unsigned)bx, (unsigned)groups);
  if (y_dtype == kDtypeF32)
    return launch_kernel(dequant_kernel<false>, grid, dim3(kThreads), 0, stream, (const uint32_t*)codes, scales, units,
                         s_g, y);
  return launch_kernel(dequant_kernel<true>, grid, dim3(kThreads), 0, stream, (const uint32_t*)codes, scales, units,
                       s_g, y);
}

}  // namespace nvfp4
